"""Benchmark of the indexer-Q preparation hot path on one MI355X.

One step = the whole path over one batch of 4,632 tokens (X bf16 [4632, 1536]):
packed-UE8M0 FP8 quantization, then the fused block-scaled FP8 Q projection +
RoPE + Hadamard-128 + FP4 kernel (64 heads x 128). Inputs are synthetic and
already resident in HBM when timing starts; outputs are preallocated.

The K timed steps are captured into one HIP graph and replayed (the eager
launch rate of the same steps is reported beside it). Prints ONE JSON line
with whole-job tokens/s, the fused kernel's MFMA roofline
(algorithmic FLOPs / measured average kernel time, against the dense FP8 peak),
the standalone quantizer's HBM roofline on a [4632, 7168] matrix (rotated over
enough buffer sets to defeat the 256 MiB Infinity Cache), and the CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

`--workload decode` instead measures the decode-shaped mix: 256 independent
calls with M drawn from {1, 2, 4, 8, 16, 32, 64} (each: the indexer-Q
preparation of X [M, 1536] in one launch, and a standalone quantization of
X' [M, 7168]), replayed from one captured HIP graph (sustained calls/s), with
per-M latencies from graphs of repeated single calls; the two-call path
(quantize, then the fused kernel) is measured beside it.

`--workload prefill32k` measures the long-prefill workload: the chain at
32,768 tokens (X Student-t, nu = 3; positions 0..32767) and the standalone
quantizer on X' [32768, 7168]. The default line also carries the standalone
epilogue (bf16 Q [4632, 64x128] -> RoPE, Hadamard, FP4) against its HBM
roofline; `--vendor-gemm` adds the vendor FP8 GEMM (hipBLASLt) timed at the
projection shape, as context only.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
M_TOKENS, K_PROJ, N_HEADS, HEAD_DIM = 4632, 1536, 64, 128
QUANT_M, QUANT_K = 4632, 7168


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: calibrate to ~15 s)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of 256 MiB (for HBM byte-counter scaling)")
    ap.add_argument("--workload", choices=("prefill", "prefill32k", "decode"), default="prefill")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor FP8 GEMM (hipBLASLt via torch._scaled_mm, per-tensor scales, "
                         "bf16 out) at the projection shape, as context for the fused kernel's MFMA fraction")
    return ap.parse_args()


def fused_bytes(M):
    """Algorithmic HBM bytes of one fused launch: A + its scale words, W + its
    scales, positions, the table rows read, and the FP4 codes + scales written."""
    nkb = K_PROJ // 128
    return (M * K_PROJ + M * 4 * ((nkb + 3) // 4) + N_HEADS * HEAD_DIM * K_PROJ + N_HEADS * nkb
            + M * 8 + M * 64 * 4 + M * N_HEADS * (HEAD_DIM // 2 + HEAD_DIM // 32))


# The sources each measured kernel is built from: a committed traffic figure is
# used only while these files hash to the digest recorded beside it.
KERNEL_SOURCES = {
    "fused": ("indexer_q_pipe.hip", "iq_common.h"),        # the K = 1536 kernel
    "quant": ("quant_fp8.hip",),
    "epilogue": ("epilogue_bf16.hip", "iq_common.h"),
}
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "indexer_q_chain_m4632_rocprofv3.md")


def source_digest(kernel):
    """First 16 hex digits of the SHA-256 of a kernel's sources."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "fp4_quantized_prep_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or None if
    the kernel's sources changed since the counters were taken."""
    try:
        fields = dict(line.strip().split(": ", 1) for line in open(TRAFFIC_PROFILE)
                      if line.strip().startswith(kernel + "_"))
        digest = source_digest(kernel)
    except (OSError, ValueError):
        return None
    if fields.get(f"{kernel}_kernel_source_sha256_16") != digest:
        return None
    return int(fields[f"{kernel}_traffic_bytes_per_launch"])


MFMA_PROFILE = os.path.join(ROOT, "profiles", "indexer_q_pipe_mfma_counters_m4632.md")


def measured_mfma_util():
    """The fused kernel's MFMA busy share (SQ_VALU_MFMA_BUSY_CYCLES over the
    SIMDs' active cycles) from the committed rocprofv3 counter summary, or
    None if the kernel's sources changed since the counters were taken."""
    try:
        fields = dict(line.strip().split(": ", 1) for line in open(MFMA_PROFILE)
                      if line.strip().startswith("fused_"))
    except (OSError, ValueError):
        return None
    if fields.get("fused_kernel_source_sha256_16") != source_digest("fused"):
        return None
    return float(fields["fused_mfma_util_pct"]) / 100.0


def one_launch_bytes(M):
    """Algorithmic HBM bytes of one one-launch call: bf16 X, W + its scales,
    positions, the table rows read, and the FP4 codes + scales written."""
    nkb = K_PROJ // 128
    return (M * K_PROJ * 2 + N_HEADS * HEAD_DIM * K_PROJ + N_HEADS * nkb + M * 8 + M * 64 * 4
            + M * N_HEADS * (HEAD_DIM // 2 + HEAD_DIM // 32))


def epilogue_bytes(M, H=N_HEADS):
    """Algorithmic HBM bytes of one standalone-epilogue launch: per (token, head)
    256 B of bf16 Q in, 64 B of codes and 4 scale bytes out; per token its
    position (8 B) and table row (64 float32)."""
    return M * H * (2 * HEAD_DIM + HEAD_DIM // 2 + HEAD_DIM // 32) + M * (8 + 64 * 4)


def quant_bytes(M, K):
    """Algorithmic HBM bytes of one quantizer launch: bf16 in, E4M3 + words out."""
    return M * K * 2 + M * K + M * 4 * ((K // 128 + 3) // 4)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no cross-GPU step); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    if args.workload == "decode":
        decode_bench(args)
        return
    if args.workload == "prefill32k":
        prefill32k_bench(args)
        return

    import numpy as np
    import torch

    import fp4_quantized_prep_amd as iqp
    import synthetic as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] device {torch.cuda.get_device_name(dev)}; preparing inputs", file=sys.stderr, flush=True)

    inp = S.indexer_q_inputs("indexer_q_m4632")
    x = inp["x"].to(dev)
    pos = inp["positions"].to(dev)
    w_cpu, wsb_cpu = S.weights()
    w, wsb = w_cpu.to(dev), wsb_cpu.to(dev)
    cs = iqp.rope_cos_sin_table(S.ROPE_THETA, inp["max_pos"], 64, device=dev)
    M = x.shape[0]
    a = torch.empty((M, K_PROJ), dtype=torch.uint8, device=dev)
    a_s = torch.empty((M, (K_PROJ // 128 + 3) // 4), dtype=torch.int32, device=dev)
    q = torch.empty((M, N_HEADS, HEAD_DIM // 2), dtype=torch.uint8, device=dev)
    qs = torch.empty((M, N_HEADS, HEAD_DIM // 32), dtype=torch.uint8, device=dev)

    def step():
        iqp.fp8_quant_1x128_ue8m0(x, q=a, scales=a_s)
        iqp.indexer_q_gemm_rope_fp4(a, a_s, w, wsb, pos, cs, n_heads=N_HEADS, q_fp4=q, q_scales=qs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- K whole steps launched one after another, as an eager caller would,
    # with events only at the two ends (an event between two kernels adds a
    # dispatch gap of its own); reported beside the timed region below
    K = args.steps
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(K):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / K
    tokens_per_s = M * K / (total_ms * 1e-3)

    # ---- timed region (`value`): the same K steps captured into one HIP graph
    # and replayed, one untimed replay, then one timed between two events on
    # the stream: every kernel of every step runs, without the host's
    # per-launch dispatch gaps
    t_step_graph = graph_launch_time(lambda i: step(), K, reps=1)
    tokens_per_s_graph = M / t_step_graph

    # ---- the same K steps again with an event pair around each kernel: each
    # kernel's average in the chain (the events' own gaps are in these figures)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        iqp.fp8_quant_1x128_ue8m0(x, q=a, scales=a_s)
        ev[i][1].record(stream)
        iqp.indexer_q_gemm_rope_fp4(a, a_s, w, wsb, pos, cs, n_heads=N_HEADS, q_fp4=q, q_scales=qs)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t_quant = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3       # s
    t_fused_ev = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    pct = lambda v: {f"p{q}": float(np.percentile(v, q)) * 1e3 for q in (10, 50, 90)}   # ms -> us
    in_chain_us = {"quant": pct([e[0].elapsed_time(e[1]) for e in ev]),
                   "fused": pct([e[1].elapsed_time(e[2]) for e in ev])}
    # the fused kernel's own duration: K launches back to back from a captured
    # graph between two events on its stream (the input A stays the chain's)
    t_fused = graph_launch_time(
        lambda i: iqp.indexer_q_gemm_rope_fp4(a, a_s, w, wsb, pos, cs, n_heads=N_HEADS, q_fp4=q, q_scales=qs),
        max(20, min(K, 100)))
    flops = 2.0 * M * (N_HEADS * HEAD_DIM) * K_PROJ
    fused_tflops = flops / t_fused / 1e12
    # context: the same projection with both convention flags (interleaved RoPE,
    # OCP floor-rule FP4 scales), the pipelined kernel's variant build
    t_variant = graph_launch_time(
        lambda i: iqp.indexer_q_gemm_rope_fp4(a, a_s, w, wsb, pos, cs, n_heads=N_HEADS, q_fp4=q, q_scales=qs,
                                              rope_layout="interleaved", scale_rule="ocp_floor"),
        max(20, min(K, 100)))
    print(f"[bench] chain from a captured graph: {t_step_graph * 1e6:.1f} us/step = {tokens_per_s_graph:.3e} tokens/s",
          file=sys.stderr, flush=True)
    print(f"[bench] chain: {ms_per_step * 1e3:.1f} us/step (wall {wall * 1e6 / K:.1f} us); "
          f"fused kernel {t_fused * 1e6:.1f} us back to back = {fused_tflops:.0f} TFLOP/s; with an event "
          f"pair around each kernel: quant {t_quant * 1e6:.1f} us, fused {t_fused_ev * 1e6:.1f} us; "
          f"with both convention flags {t_variant * 1e6:.1f} us", file=sys.stderr, flush=True)

    # ---- standalone quantizer on [4632, 7168], rotating buffer sets (> 256 MiB)
    xq_cpu = S.quant_input("quant_4632x7168")
    n_sets = 5
    xs = [xq_cpu.to(dev) for _ in range(n_sets)]
    qq = [torch.empty((QUANT_M, QUANT_K), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    ss = [torch.empty((QUANT_M, (QUANT_K // 128 + 3) // 4), dtype=torch.int32, device=dev) for _ in range(n_sets)]
    for i in range(10):
        iqp.fp8_quant_1x128_ue8m0(xs[i % n_sets], q=qq[i % n_sets], scales=ss[i % n_sets])
    torch.cuda.synchronize()
    # Launches replayed back to back from a captured graph between two events on
    # the kernel's stream, so the average is the kernel's own duration (an event
    # pair around every launch adds ~2.5 us of dispatch gap at this size); the
    # per-launch-event figure is reported beside it.
    n_q = max(50, K)
    t_q_big = graph_launch_time(
        lambda i: iqp.fp8_quant_1x128_ue8m0(xs[i % n_sets], q=qq[i % n_sets], scales=ss[i % n_sets]), n_q)
    qev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_q)]
    for i in range(n_q):
        k = i % n_sets
        qev[i][0].record(stream)
        iqp.fp8_quant_1x128_ue8m0(xs[k], q=qq[k], scales=ss[k])
        qev[i][1].record(stream)
    torch.cuda.synchronize()
    t_q_ev = float(np.mean([b.elapsed_time(e) for b, e in qev])) * 1e-3
    qbytes = quant_bytes(QUANT_M, QUANT_K)
    q_gbs = qbytes / t_q_big / 1e9
    print(f"[bench] quantizer [4632,7168]: {t_q_big * 1e6:.1f} us = {q_gbs:.0f} GB/s back to back (graph); "
          f"{t_q_ev * 1e6:.1f} us with an event pair around each launch", file=sys.stderr, flush=True)
    del xs, qq, ss

    # ---- standalone epilogue (bf16 Q -> RoPE, Hadamard, FP4) on [4632, 64*128],
    # rotating buffer sets (> 256 MiB), launches back to back
    qin = S.q_bf16_inputs("indexer_q_m4632")
    e_sets = 4
    eq = [qin["q"].to(dev) for _ in range(e_sets)]
    eo = [torch.empty((M, N_HEADS, HEAD_DIM // 2), dtype=torch.uint8, device=dev) for _ in range(e_sets)]
    es = [torch.empty((M, N_HEADS, HEAD_DIM // 32), dtype=torch.uint8, device=dev) for _ in range(e_sets)]
    for i in range(8):
        iqp.indexer_q_rope_hadamard_fp4(eq[i % e_sets], pos, cs, n_heads=N_HEADS, q_fp4=eo[i % e_sets],
                                        q_scales=es[i % e_sets])
    torch.cuda.synchronize()
    n_e = max(40, K)
    t_epi = graph_launch_time(
        lambda i: iqp.indexer_q_rope_hadamard_fp4(eq[i % e_sets], pos, cs, n_heads=N_HEADS, q_fp4=eo[i % e_sets],
                                                  q_scales=es[i % e_sets]), n_e)
    ebytes = epilogue_bytes(M)
    e_gbs = ebytes / t_epi / 1e9
    print(f"[bench] standalone epilogue [4632, 64x128] bf16: {t_epi * 1e6:.1f} us = {e_gbs:.0f} GB/s",
          file=sys.stderr, flush=True)
    del eq, eo, es

    # ---- weight preparation (off the per-token path): bf16 W [8192, 1536] ->
    # E4M3 + 128x128 UE8M0, 10 rotating sets (376 MB), graph-replayed
    wg = np.random.default_rng([100, 1])
    wb = torch.from_numpy((wg.standard_normal((N_HEADS * HEAD_DIM, K_PROJ)) * 0.02).astype(np.float32)).to(
        torch.bfloat16)
    w_sets = 10
    wbs = [wb.to(dev) for _ in range(w_sets)]
    wqs = [torch.empty((N_HEADS * HEAD_DIM, K_PROJ), dtype=torch.uint8, device=dev) for _ in range(w_sets)]
    wss = [torch.empty((N_HEADS * HEAD_DIM // 128, K_PROJ // 128), dtype=torch.uint8, device=dev)
           for _ in range(w_sets)]
    t_wq = graph_launch_time(lambda i: iqp.fp8_quant_weight_128x128_ue8m0(
        wbs[i % w_sets], q=wqs[i % w_sets], scales=wss[i % w_sets]), 40)
    wq_bytes = N_HEADS * HEAD_DIM * K_PROJ * 3 + (N_HEADS * HEAD_DIM // 128) * (K_PROJ // 128)
    print(f"[bench] weight preparation [8192, 1536]: {t_wq * 1e6:.1f} us = {wq_bytes / t_wq / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)
    del wbs, wqs, wss

    vendor = vendor_gemm_context(M, dev) if args.vendor_gemm else None

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_tokens, inp, w_cpu, wsb_cpu)

    result = {
        "metric": "tokens/sec & % roofline: FP8 quant (HBM GB/s) + fused indexer-Q (MFMA util)",
        "value": tokens_per_s_graph,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": t_step_graph * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate), bf16 in, fp4-e2m1 out",
        "data": "synthetic",
        "config": {
            "workload": "indexer-Q chain, 4632 tokens: X bf16 [4632,1536] -> FP8 1x128 UE8M0 -> "
                        "Q = A W^T (W [8192,1536] E4M3, 128x128 UE8M0) -> RoPE(64 of 128) -> "
                        "Hadamard-128 -> FP4 e2m1 [4632,64,64] + UE8M0 [4632,64,4]",
            "tokens": M, "K": K_PROJ, "heads": N_HEADS, "head_dim": HEAD_DIM, "rope_dim": 64,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "indexer_q_pipe_kernel (fused GEMM + RoPE + Hadamard + FP4; launches back to back from a "
                      "captured graph on the chain's A)",
            "bound": "mfma",
            "achieved": fused_tflops,
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": fused_tflops / PEAK_FP8_TFLOPS,
            "traffic": measured_traffic("fused"),
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": t_fused * 1e6,
            "avg_launch_us_event_pair_each": t_fused_ev * 1e6,
            "avg_launch_us_interleaved_rope_ocp_floor_scales": t_variant * 1e6,
            "mfma_busy_frac_counters": measured_mfma_util(),
        },
        "quant_roofline": {
            "kernel": "fp8_quant_1x128_kernel on [4632,7168] (5 rotating buffer sets, launches back to back "
                      "from a captured graph)",
            "bound": "hbm",
            "achieved": q_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": q_gbs / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": qbytes,
            "traffic": measured_traffic("quant"),
            "avg_launch_us": t_q_big * 1e6,
            "avg_launch_us_event_pair_each": t_q_ev * 1e6,
            "in_chain_avg_launch_us": t_quant * 1e6,
        },
        "epilogue_roofline": {
            "kernel": "indexer_q_epilogue_kernel (bf16 Q [4632, 64x128] -> RoPE, Hadamard-128, FP4; "
                      "4 rotating buffer sets, launches back to back from a captured graph)",
            "bound": "hbm",
            "achieved": e_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": e_gbs / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": ebytes,
            "traffic": measured_traffic("epilogue"),
            "avg_launch_us": t_epi * 1e6,
        },
        "weight_prep_roofline": {
            "kernel": "fp8_quant_weight_kernel (bf16 W [8192,1536] -> E4M3 + 128x128 UE8M0; off the per-token "
                      "path; 10 rotating sets, graph-replayed)",
            "bound": "hbm",
            "achieved": wq_bytes / t_wq / 1e9,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": wq_bytes / t_wq / 1e9 / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": wq_bytes,
            "avg_launch_us": t_wq * 1e6,
        },
        "cpu_baseline": cpu,
        "in_chain_kernel_us": in_chain_us,
        "timing": "K whole steps captured into one HIP graph, one untimed replay, then one replay between two "
                  "events on the stream (synchronized before and after)",
        "eager": {"ms_per_step": ms_per_step, "tokens_per_s": tokens_per_s,
                  "note": "the same K steps launched one after another from Python, events only at the ends"},
        "runtime": {"hip": torch.version.hip, "torch": torch.__version__,
                    "device": torch.cuda.get_device_name(dev)},
    }
    if vendor is not None:
        result["vendor_gemm_context"] = vendor
    print(json.dumps(result), flush=True)


def graph_launch_time(launch, n_calls, reps=5):
    """Average device time per call of launch(0..n_calls-1), replayed from one
    captured HIP graph between two events on the current stream: host-side
    launch cost (the Python binding's checks) is out of the measurement, so a
    short kernel is not starved by its own launches."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / (reps * n_calls)


def vendor_gemm_context(M, dev, reps=100):
    """The vendor FP8 GEMM at the projection shape [M, 1536] x [8192, 1536]^T:
    hipBLASLt through torch._scaled_mm with per-tensor scales and a bf16 output,
    no epilogue. Not part of the path: a reference for what a plain library GEMM
    reaches on this chip at this shape."""
    import torch
    x = torch.randn(M, K_PROJ, device=dev).to(torch.float8_e4m3fn)
    w = torch.randn(N_HEADS * HEAD_DIM, K_PROJ, device=dev).to(torch.float8_e4m3fn)
    one = torch.tensor(1.0, device=dev)
    fn = lambda: torch._scaled_mm(x, w.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
    for _ in range(10):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    tflops = 2.0 * M * N_HEADS * HEAD_DIM * K_PROJ / us * 1e-6
    print(f"[bench] vendor FP8 GEMM (hipBLASLt, per-tensor scales, bf16 out): {us:.1f} us = {tflops:.0f} TFLOP/s",
          file=sys.stderr, flush=True)
    return {"what": "torch._scaled_mm (hipBLASLt) e4m3 [M,1536] x [8192,1536]^T, per-tensor scales, bf16 out, "
                    "no epilogue; launches back to back", "avg_launch_us": us, "achieved_tflops": tflops,
            "frac": tflops / PEAK_FP8_TFLOPS}


def prefill32k_bench(args):
    """The long-prefill workload: the chain at 32,768 tokens (X Student-t nu=3,
    positions 0..32767) and the standalone quantizer on X' [32768, 7168];
    prints one JSON line in the same form as the default workload."""
    import numpy as np
    import torch

    import fp4_quantized_prep_amd as iqp
    import synthetic as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    inp = S.indexer_q_inputs("prefill_m32768")
    x, pos = inp["x"].to(dev), inp["positions"].to(dev)
    w_cpu, wsb_cpu = S.weights()
    w, wsb = w_cpu.to(dev), wsb_cpu.to(dev)
    cs = iqp.rope_cos_sin_table(S.ROPE_THETA, inp["max_pos"], 64, device=dev)
    M = x.shape[0]
    a = torch.empty((M, K_PROJ), dtype=torch.uint8, device=dev)
    a_s = torch.empty((M, (K_PROJ // 128 + 3) // 4), dtype=torch.int32, device=dev)
    q = torch.empty((M, N_HEADS, HEAD_DIM // 2), dtype=torch.uint8, device=dev)
    qs = torch.empty((M, N_HEADS, HEAD_DIM // 32), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        iqp.fp8_quant_1x128_ue8m0(x, q=a, scales=a_s)
        iqp.indexer_q_gemm_rope_fp4(a, a_s, w, wsb, pos, cs, n_heads=N_HEADS, q_fp4=q, q_scales=qs)
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        iqp.fp8_quant_1x128_ue8m0(x, q=a, scales=a_s)
        ev[i][1].record(stream)
        iqp.indexer_q_gemm_rope_fp4(a, a_s, w, wsb, pos, cs, n_heads=N_HEADS, q_fp4=q, q_scales=qs)
        ev[i][2].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    t_quant = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    t_fused = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    flops = 2.0 * M * (N_HEADS * HEAD_DIM) * K_PROJ
    fused_tflops = flops / t_fused / 1e12
    def step32k(i):
        iqp.fp8_quant_1x128_ue8m0(x, q=a, scales=a_s)
        iqp.indexer_q_gemm_rope_fp4(a, a_s, w, wsb, pos, cs, n_heads=N_HEADS, q_fp4=q, q_scales=qs)

    t_step_graph = graph_launch_time(step32k, K, reps=1)   # the timed `value`, as in the default workload
    print(f"[bench] chain at {M} tokens from a captured graph: {t_step_graph * 1e6:.1f} us/step",
          file=sys.stderr, flush=True)
    print(f"[bench] chain at {M} tokens: {total_ms / K * 1e3:.1f} us/step; quant {t_quant * 1e6:.1f} us, "
          f"fused {t_fused * 1e6:.1f} us = {fused_tflops:.0f} TFLOP/s", file=sys.stderr, flush=True)
    del a, a_s, q, qs

    xw_cpu = S.quant_input("prefill_m32768")
    n_sets = 2        # 2 x (470 MB in + 235 MB out): beyond the 256 MiB cache
    xs = [xw_cpu.to(dev) for _ in range(n_sets)]
    qq = [torch.empty((M, QUANT_K), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    ss = [torch.empty((M, (QUANT_K // 128 + 3) // 4), dtype=torch.int32, device=dev) for _ in range(n_sets)]
    for i in range(4):
        iqp.fp8_quant_1x128_ue8m0(xs[i % n_sets], q=qq[i % n_sets], scales=ss[i % n_sets])
    torch.cuda.synchronize()
    n_q = max(20, K // 4)
    t_qw = graph_launch_time(
        lambda i: iqp.fp8_quant_1x128_ue8m0(xs[i % n_sets], q=qq[i % n_sets], scales=ss[i % n_sets]), n_q, reps=2)
    qbytes = quant_bytes(M, QUANT_K)
    q_gbs = qbytes / t_qw / 1e9
    print(f"[bench] quantizer [{M},{QUANT_K}]: {t_qw * 1e6:.1f} us = {q_gbs:.0f} GB/s", file=sys.stderr, flush=True)
    del xs, qq, ss

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_tokens, inp, w_cpu, wsb_cpu)
    result = {
        "metric": "tokens/sec & % roofline: FP8 quant (HBM GB/s) + fused indexer-Q (MFMA util)",
        "value": M / t_step_graph,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": t_step_graph * 1e3,
        "timing": "K whole steps captured into one HIP graph, one untimed replay, then one timed",
        "eager_with_kernel_events": {"ms_per_step": total_ms / K, "tokens_per_s": M * K / (total_ms * 1e-3)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate), bf16 in, fp4-e2m1 out",
        "data": "synthetic",
        "config": {
            "workload": "long prefill, 32768 tokens: X bf16 [32768,1536] Student-t nu=3 -> FP8 1x128 UE8M0 -> "
                        "fused Q projection + RoPE + Hadamard-128 + FP4; plus the standalone quantizer on "
                        "X' [32768,7168]",
            "tokens": M, "K": K_PROJ, "heads": N_HEADS, "head_dim": HEAD_DIM, "rope_dim": 64,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "indexer_q_pipe_kernel (fused GEMM + RoPE + Hadamard + FP4; launches back to back from a "
                      "captured graph on the chain's A)",
            "bound": "mfma",
            "achieved": fused_tflops,
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": fused_tflops / PEAK_FP8_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": t_fused * 1e6,
        },
        "quant_roofline": {
            "kernel": f"fp8_quant_1x128_kernel on [{M},{QUANT_K}] (2 rotating buffer sets, launches back to back "
                      "from a captured graph)",
            "bound": "hbm",
            "achieved": q_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": q_gbs / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": qbytes,
            "avg_launch_us": t_qw * 1e6,
            "in_chain_avg_launch_us": t_quant * 1e6,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def decode_bench(args):
    """The decode-shaped mix (see the module docstring); prints one JSON line."""
    import numpy as np
    import torch

    import fp4_quantized_prep_amd as iqp
    import synthetic as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w_cpu, wsb_cpu = S.weights()
    w, wsb = w_cpu.to(dev), wsb_cpu.to(dev)
    max_pos = 131072
    cs = iqp.rope_cos_sin_table(S.ROPE_THETA, max_pos, 64, device=dev)
    calls = []
    for c in S.decode_calls(256):
        m = c["x"].shape[0]
        calls.append({
            "M": m, "x": c["x"].to(dev), "xw": c["x_wide"].to(dev), "pos": c["positions"].to(dev),
            "a": torch.empty((m, K_PROJ), dtype=torch.uint8, device=dev),
            "as": torch.empty((m, 3), dtype=torch.int32, device=dev),
            "aw": torch.empty((m, QUANT_K), dtype=torch.uint8, device=dev),
            "asw": torch.empty((m, (QUANT_K // 128 + 3) // 4), dtype=torch.int32, device=dev),
            "q": torch.empty((m, N_HEADS, HEAD_DIM // 2), dtype=torch.uint8, device=dev),
            "qs": torch.empty((m, N_HEADS, HEAD_DIM // 32), dtype=torch.uint8, device=dev),
        })

    def two(c, wt=(w, wsb)):
        # two calls: quantize, then the fused projection
        iqp.fp8_quant_1x128_ue8m0(c["x"], q=c["a"], scales=c["as"])
        iqp.indexer_q_gemm_rope_fp4(c["a"], c["as"], wt[0], wt[1], c["pos"], cs, n_heads=N_HEADS,
                                    q_fp4=c["q"], q_scales=c["qs"])
        iqp.fp8_quant_1x128_ue8m0(c["xw"], q=c["aw"], scales=c["asw"])

    def one(c, wt=(w, wsb)):
        # one launch from bf16 X to FP4 Q
        iqp.indexer_q_prep_bf16(c["x"], wt[0], wt[1], c["pos"], cs, n_heads=N_HEADS, q_fp4=c["q"],
                                q_scales=c["qs"])
        iqp.fp8_quant_1x128_ue8m0(c["xw"], q=c["aw"], scales=c["asw"])

    def routed(c, wt=(w, wsb)):
        # the serving policy: one launch up to ONE_LAUNCH_MAX_TOKENS tokens, two calls above
        (one if c["M"] <= iqp.ONE_LAUNCH_MAX_TOKENS else two)(c, wt)

    def graph_of(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def replay_time(g, reps):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps    # s per replay

    for c in calls:
        two(c)
        one(c)
    torch.cuda.synchronize()
    print(f"[bench] decode mix: {len(calls)} calls, M histogram "
          f"{ {int(m): int(n) for m, n in zip(*np.unique([c['M'] for c in calls], return_counts=True))} }",
          file=sys.stderr, flush=True)

    # sustained: the whole mix as one graph, one-launch path and two-call path
    reps = max(5, args.steps // 20)
    t_mix = replay_time(graph_of(lambda: [routed(c) for c in calls]), reps)
    t_mix1 = replay_time(graph_of(lambda: [one(c) for c in calls]), reps)
    t_mix2 = replay_time(graph_of(lambda: [two(c) for c in calls]), reps)
    calls_per_s = len(calls) / t_mix
    print(f"[bench] mix: {calls_per_s:.0f} calls/s routed (one launch up to {iqp.ONE_LAUNCH_MAX_TOKENS} tokens), "
          f"{len(calls) / t_mix1:.0f} one launch, {len(calls) / t_mix2:.0f} two calls", file=sys.stderr, flush=True)
    # cold weights: call i reads weight copy i % n_w, 24 copies of 12.6 MB (302 MB, beyond the
    # 256 MiB Infinity Cache), so every call's W streams from HBM
    n_w = 24
    w_sets = [(w.clone(), wsb.clone()) for _ in range(n_w)]
    t_cold = replay_time(graph_of(lambda: [routed(c, w_sets[i % n_w]) for i, c in enumerate(calls)]), reps)
    del w_sets
    print(f"[bench] mix with cold weights ({n_w} rotating copies): {len(calls) / t_cold:.0f} calls/s routed",
          file=sys.stderr, flush=True)

    # per-M latency of one call (the indexer-Q preparation + the wide quantization),
    # and of the indexer-Q kernel(s) alone
    lat, lat2, lat_k, lat_k2 = {}, {}, {}, {}
    n_rep = 20
    for m in sorted({c["M"] for c in calls}):
        c = next(c for c in calls if c["M"] == m)
        lat[m] = replay_time(graph_of(lambda: [one(c) for _ in range(n_rep)]), 5) / n_rep * 1e6
        lat2[m] = replay_time(graph_of(lambda: [two(c) for _ in range(n_rep)]), 5) / n_rep * 1e6
        lat_k[m] = replay_time(graph_of(lambda: [iqp.indexer_q_prep_bf16(
            c["x"], w, wsb, c["pos"], cs, n_heads=N_HEADS, q_fp4=c["q"], q_scales=c["qs"])
            for _ in range(n_rep)]), 5) / n_rep * 1e6
        lat_k2[m] = replay_time(graph_of(lambda: [iqp.indexer_q_gemm_rope_fp4(
            c["a"], c["as"], w, wsb, c["pos"], cs, n_heads=N_HEADS, q_fp4=c["q"], q_scales=c["qs"])
            for _ in range(n_rep)]), 5) / n_rep * 1e6
        print(f"[bench] M={m}: call {lat[m]:.2f} us one launch ({lat_k[m]:.2f} us kernel), "
              f"{lat2[m]:.2f} us two calls ({lat_k2[m]:.2f} us fused kernel)", file=sys.stderr, flush=True)
    per_call = np.array([(lat if c["M"] <= iqp.ONE_LAUNCH_MAX_TOKENS else lat2)[c["M"]] for c in calls])
    per_call1 = np.array([lat[c["M"]] for c in calls])
    per_call2 = np.array([lat2[c["M"]] for c in calls])
    # the one-launch kernel reads bf16 X and all of W (and its scales) once per
    # call; W dominates its algorithmic bytes at these sizes: its bound is HBM
    mix_bytes = float(sum(one_launch_bytes(c["M"]) for c in calls))
    mix_k_s = float(sum(lat_k[c["M"]] for c in calls)) * 1e-6
    mean_k = mix_k_s / len(calls) * 1e6
    achieved = mix_bytes / mix_k_s / 1e9
    result = {
        "metric": "decode-shaped indexer-Q calls/s (graph replay)",
        "value": calls_per_s,
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": 1,
        "ms_per_step": t_mix * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate), bf16 in, fp4-e2m1 out",
        "data": "synthetic",
        "config": {
            "workload": "decode mix: 256 independent calls, M uniform over {1,2,4,8,16,32,64}; each call "
                        "X bf16 [M,1536] -> FP8 quant -> GEMM + RoPE + Hadamard + FP4 (64 heads), one launch "
                        "up to 16 tokens and two calls above, plus a standalone FP8 quant of X' [M,7168]; "
                        "positions U[0,131072)",
            "calls": len(calls), "K": K_PROJ, "heads": N_HEADS, "head_dim": HEAD_DIM, "max_pos": max_pos,
            "parallelism": "single GPU",
        },
        "latency_us": {"p50": float(np.percentile(per_call, 50)), "p99": float(np.percentile(per_call, 99))},
        "cold_weights": {"calls_per_s": len(calls) / t_cold, "weight_copies": n_w,
                         "note": "routed mix, call i reads weight copy i % 24 (302 MB, beyond the Infinity Cache)"},
        "one_launch_path": {"calls_per_s": len(calls) / t_mix1,
                            "p50_us": float(np.percentile(per_call1, 50)),
                            "p99_us": float(np.percentile(per_call1, 99)),
                            "per_M_call": {str(k): v for k, v in lat.items()},
                            "per_M_kernel": {str(k): v for k, v in lat_k.items()}},
        "two_call_path": {"calls_per_s": len(calls) / t_mix2,
                          "p50_us": float(np.percentile(per_call2, 50)),
                          "p99_us": float(np.percentile(per_call2, 99)),
                          "per_M_call": {str(k): v for k, v in lat2.items()},
                          "per_M_fused_kernel": {str(k): v for k, v in lat_k2.items()}},
        "roofline": {
            "kernel": "indexer_q_small_kernel<bf16 in> (FP8 quant + GEMM + RoPE + Hadamard + FP4, M <= 256)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": None,
            "algorithmic_bytes_per_launch": mix_bytes / len(calls),
            "avg_launch_us": mean_k,
        },
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(n_tokens, inp, w_cpu, wsb_cpu):
    """Time the oracle (as it stands) on the first n tokens of the workload:
    its FP8 quantization and its whole fused chain."""
    import numpy as np

    from oracle import indexer_q as IQ
    from oracle import quant_fp8 as QO

    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))

    x = inp["x"].float().numpy()
    pos = inp["positions"].numpy()
    w = w_cpu.numpy()
    wsb = wsb_cpu.numpy()

    def run(n):
        t0 = time.perf_counter()
        a, words = QO.fp8_quant_1x128_ue8m0(x[:n])
        IQ.indexer_q_chain(a, QO.unpack_scale_words(words, K_PROJ // 128), w, wsb, pos[:n], n_heads=N_HEADS)
        return time.perf_counter() - t0

    # about 15 s of CPU work: a prefix of the tokens if one pass is slower
    # than that, else the whole batch repeated
    target = 15.0
    reps = 1
    total = x.shape[0]
    if n_tokens <= 0:
        est_full = run(128) * total / 128
        if est_full > target:
            n_tokens = int(max(128, total * target / est_full))
        else:
            n_tokens = total
            reps = max(1, int(round(target / max(est_full, 1e-3))))
    dt = sum(run(n_tokens) for _ in range(reps))
    print(f"[bench] oracle: {reps} x {n_tokens} tokens in {dt:.2f} s on {threads} threads", file=sys.stderr, flush=True)
    return {"value": reps * n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} pass(es) over the first {n_tokens} of the {total} tokens, whole chain (quantize + "
                      f"GEMM + RoPE + Hadamard + FP4), numpy float64, {dt:.1f} s"}


if __name__ == "__main__":
    main()
