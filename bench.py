"""Benchmark of the indexer-Q preparation hot path on one MI355X.

One step = the whole path over one batch of tokens (X bf16 [M, 1536]):
packed-UE8M0 FP8 quantization, then the fused block-scaled FP8 Q projection +
RoPE + Hadamard-128 + FP4 kernel (64 heads x 128). Inputs are synthetic and
already resident in HBM when timing starts; outputs are preallocated. Like the
weights, the RoPE table and its lane-ordered copy (which the prefill kernel
reads; the same values rearranged for its 16-byte loads) are built once
before timing.

The headline `value` is the 4,632-token chain (tokens/s). Every chain config
(128, 4,632 and 32,768 tokens) is timed the way the TensorRT-LLM PR page
(Description / Results) times its paths: K steps captured into one HIP graph,
the graph replayed R times with an event pair around each replay, the median
replay taken; the configs run once in forward and once in reverse order and
the two medians are averaged. p10 / p90 over all 2R replays are reported
beside. The same line carries:

* the fused kernel's MFMA roofline (algorithmic FLOPs / median kernel time
  against the 5.0 PFLOP/s dense FP8 spec), and the shader clock it ran at,
  read from the kernel's clock-stamp build (s_memtime / s_memrealtime deltas
  per workgroup), with the fraction against the peak scaled to that clock;
* the standalone quantizer's HBM roofline on X' [4632, 7168] and on
  X' [32768, 7168] (rotated over enough buffer sets to defeat the 256 MiB
  Infinity Cache), beside a plain device copy's rate;
* the decode-shaped mix: 256 independent calls with M from {1, 2, 4, 8, 16,
  32, 64}, sustained calls/s from one captured graph, with hot and cold
  (rotating) weights, and per-call latency percentiles;
* the standalone epilogue and the weight preparation against HBM;
* the CPU oracle timed on a bounded sample of the 4,632-token workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

`--workload` picks one part alone (for profiling runs): `prefill` (the
4,632-token chain), `prefill128`, `prefill32k`, `decode`; `all` (default) is
the whole line. `--vendor-gemm` adds the vendor FP8 GEMM (hipBLASLt) timed at
the projection shape, as context only.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, TFLOP/s, at the 2.4 GHz peak clock
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
K_PROJ, N_HEADS, HEAD_DIM = 1536, 64, 128
QUANT_K = 7168
W_BYTES = N_HEADS * HEAD_DIM * K_PROJ + N_HEADS * (K_PROJ // 128)   # E4M3 weights + tile scales

# chain configs: name -> (tokens, synthetic workload)
CHAINS = {
    "c0_chain_m128": (128, "indexer_q_m128"),
    "c2_chain_m4632": (4632, "indexer_q_m4632"),
    "c4_chain_m32768": (32768, "prefill_m32768"),
}
HEADLINE = "c2_chain_m4632"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="steps per captured graph (one replay)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replays", type=int, default=10, help="timed replays per config and order (>= 5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: calibrate to ~15 s)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of 256 MiB (for HBM byte-counter scaling)")
    ap.add_argument("--workload", choices=("all", "prefill", "prefill128", "prefill32k", "decode"), default="all")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor FP8 GEMM (hipBLASLt via torch._scaled_mm, per-tensor scales, "
                         "bf16 out) at the projection shape, as context for the fused kernel's MFMA fraction")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work per launch

def fused_flops(M):
    return 2.0 * M * (N_HEADS * HEAD_DIM) * K_PROJ


def fused_bytes(M):
    """Algorithmic HBM bytes of one fused launch: A + its scale words, W + its
    scales, positions, the table rows read, and the FP4 codes + scales written."""
    nkb = K_PROJ // 128
    return (M * K_PROJ + M * 4 * ((nkb + 3) // 4) + W_BYTES + M * 8 + M * 64 * 4
            + M * N_HEADS * (HEAD_DIM // 2 + HEAD_DIM // 32))


def one_launch_bytes(M):
    """Algorithmic HBM bytes of one one-launch call: bf16 X, W + its scales,
    positions, the table rows read, and the FP4 codes + scales written."""
    return M * K_PROJ * 2 + W_BYTES + M * 8 + M * 64 * 4 + M * N_HEADS * (HEAD_DIM // 2 + HEAD_DIM // 32)


def epilogue_bytes(M, H=N_HEADS):
    """Algorithmic HBM bytes of one standalone-epilogue launch: per (token, head)
    256 B of bf16 Q in, 64 B of codes and 4 scale bytes out; per token its
    position (8 B) and table row (64 float32)."""
    return M * H * (2 * HEAD_DIM + HEAD_DIM // 2 + HEAD_DIM // 32) + M * (8 + 64 * 4)


def quant_bytes(M, K):
    """Algorithmic HBM bytes of one quantizer launch: bf16 in, E4M3 + words out."""
    return M * K * 2 + M * K + M * 4 * ((K // 128 + 3) // 4)


# ---------------------------------------------------------------------------
# committed counter figures (used only while the kernel sources are unchanged)

KERNEL_SOURCES = {
    "fused": ("indexer_q_pipe.hip", "indexer_q_split_lanes.hip", "iq_common.h"),   # the split-role kernel
    "quant": ("quant_fp8.hip", "fp8_block.h"),
    "epilogue": ("epilogue_bf16.hip", "iq_common.h"),
}
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "indexer_q_chain_m4632_rocprofv3.md")
MFMA_PROFILE = os.path.join(ROOT, "profiles", "indexer_q_split_lanes_mfma_counters_m4632.md")


def source_digest(kernel):
    """First 16 hex digits of the SHA-256 of a kernel's sources."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "fp4_quantized_prep_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _profile_fields(path, prefix):
    try:
        return dict(line.strip().split(": ", 1) for line in open(path) if line.strip().startswith(prefix))
    except (OSError, ValueError):
        return {}


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or None if
    the kernel's sources changed since the counters were taken."""
    fields = _profile_fields(TRAFFIC_PROFILE, kernel + "_")
    if fields.get(f"{kernel}_kernel_source_sha256_16") != source_digest(kernel):
        return None
    return int(fields[f"{kernel}_traffic_bytes_per_launch"])


def measured_mfma_util():
    """The fused kernel's MFMA busy share from the committed rocprofv3 counter
    summary, or None if the kernel's sources changed since."""
    fields = _profile_fields(MFMA_PROFILE, "fused_")
    if fields.get("fused_kernel_source_sha256_16") != source_digest("fused"):
        return None
    return float(fields["fused_mfma_util_pct"]) / 100.0


# ---------------------------------------------------------------------------
# timing helpers

def capture(launch, n_calls):
    """One HIP graph of launch(0..n_calls-1), captured after one eager call on
    a side stream."""
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
    torch.cuda.synchronize()
    return g


def replay_times(g, n_calls, reps):
    """Per-call device time (s) of each of `reps` replays of g, each between an
    event pair on the current stream, after one untimed replay."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 / n_calls for a, b in ev]


def stats_us(samples):
    import numpy as np
    s = np.asarray(samples) * 1e6
    return {"p10_us": float(np.percentile(s, 10)), "p50_us": float(np.percentile(s, 50)),
            "p90_us": float(np.percentile(s, 90)), "n": int(s.size)}


def graph_launch_time(launch, n_calls, reps=5):
    """Median per-call device time (s) of launch(0..n_calls-1) replayed from
    one captured graph (host launch cost out of the measurement), and the
    per-replay samples."""
    import numpy as np
    t = replay_times(capture(launch, n_calls), n_calls, reps)
    return float(np.median(t)), t


# ---------------------------------------------------------------------------
# the chain configs

class Chain:
    """Inputs, preallocated outputs and the step of one chain config."""

    def __init__(self, iqp, S, dev, w, wsb, tables, name):
        import torch
        M, workload = CHAINS[name]
        inp = S.indexer_q_inputs(workload)
        assert inp["x"].shape[0] == M
        self.name, self.M, self.iqp = name, M, iqp
        self.inp = inp
        self.x = inp["x"].to(dev)
        self.pos = inp["positions"].to(dev)
        self.w, self.wsb = w, wsb
        if inp["max_pos"] not in tables:
            cs = iqp.rope_cos_sin_table(S.ROPE_THETA, inp["max_pos"], 64, device=dev)
            tables[inp["max_pos"]] = (cs, iqp.rope_table_lanes(cs))
        # the table and its lane-ordered copy, both built once per table (like the weights)
        self.cs, self.cs_lanes = tables[inp["max_pos"]]
        self.a = torch.empty((M, K_PROJ), dtype=torch.uint8, device=dev)
        self.a_s = torch.empty((M, (K_PROJ // 128 + 3) // 4), dtype=torch.int32, device=dev)
        self.q = torch.empty((M, N_HEADS, HEAD_DIM // 2), dtype=torch.uint8, device=dev)
        self.qs = torch.empty((M, N_HEADS, HEAD_DIM // 32), dtype=torch.uint8, device=dev)

    def quant(self):
        self.iqp.fp8_quant_1x128_ue8m0(self.x, q=self.a, scales=self.a_s)

    def fused(self):
        self.iqp.indexer_q_gemm_rope_fp4(self.a, self.a_s, self.w, self.wsb, self.pos, self.cs, n_heads=N_HEADS,
                                         q_fp4=self.q, q_scales=self.qs, cos_sin_lanes=self.cs_lanes)

    def step(self, i=0):
        self.quant()
        self.fused()


def steps_for(M, K):
    """Steps per replay: K at the headline size, scaled so one replay of a
    config stays between about 2 and 20 ms."""
    return int(min(max(K * 4632 // max(M, 1), 20), 1000)) if M != 4632 else K


def time_chains(chains, K, reps):
    """Forward then reverse order over the chain configs: per config, its
    graph of steps_for(M, K) steps replayed `reps` times in each order."""
    import numpy as np
    graphs = {n: (capture(c.step, steps_for(c.M, K)), steps_for(c.M, K)) for n, c in chains.items()}
    order = list(chains)
    res = {n: {"forward": [], "reverse": []} for n in order}
    for direction, seq in (("forward", order), ("reverse", order[::-1])):
        for n in seq:
            g, k = graphs[n]
            res[n][direction] = replay_times(g, k, reps)
    out = {}
    for n in order:
        f, r = res[n]["forward"], res[n]["reverse"]
        med = 0.5 * (float(np.median(f)) + float(np.median(r)))
        out[n] = {"step_s": med, "forward_median_us": float(np.median(f)) * 1e6,
                  "reverse_median_us": float(np.median(r)) * 1e6, "steps_per_replay": graphs[n][1],
                  "spread": stats_us(f + r)}
    return out, order


def fused_alone(c, reps):
    """The fused kernel's own duration: launches back to back from a captured
    graph on the chain's A."""
    n = max(20, min(200, 400_000 // max(c.M, 1)))
    t, samples = graph_launch_time(lambda i: c.fused(), n, reps)
    return t, samples


def clock_during(c, iqp, n_launch=30):
    """Mean shader clock during the fused kernel: the clock-stamp build of the
    split-role kernel launched n_launch times back to back on the chain's A;
    per launch, (sum of s_memtime deltas) / (sum of s_memrealtime deltas) x the
    counter rate over its workgroups; the median of the last two thirds."""
    import numpy as np
    import torch
    wall_hz, peak_hz = iqp.device_clock_rates()
    stamps = torch.zeros((n_launch, 4 * 4096), dtype=torch.int64, device=c.x.device)
    views = []
    for i in range(n_launch):
        _, _, st = iqp.debug_indexer_q_clock(c.a, c.a_s, c.w, c.wsb, c.pos, c.cs, q_fp4=c.q, q_scales=c.qs,
                                             stamps=stamps[i], cos_sin_lanes=c.cs_lanes)
        views.append(st)
    torch.cuda.synchronize()
    clocks = []
    for st in views:
        s = st.cpu().numpy().astype(np.float64)
        live = s[:, 3] != 0
        clocks.append((s[live, 1] - s[live, 0]).sum() / (s[live, 3] - s[live, 2]).sum() * wall_hz)
    tail = clocks[n_launch // 3:]
    return {"sclk_ghz": float(np.median(tail)) / 1e9, "sclk_ghz_p10": float(np.percentile(tail, 10)) / 1e9,
            "sclk_ghz_p90": float(np.percentile(tail, 90)) / 1e9, "peak_sclk_ghz": peak_hz / 1e9,
            "counter_mhz": wall_hz / 1e6,
            "method": f"clock-stamp build of the split-role kernel, {n_launch} launches back to back on the "
                      "chain's A; per launch sum(s_memtime deltas) / sum(s_memrealtime deltas) x counter rate "
                      "over its workgroups; median of the last two thirds"}


def fused_roofline(M, t_fused, samples, clock, name):
    ach = fused_flops(M) / t_fused / 1e12
    r = {"kernel": name, "bound": "mfma", "achieved": ach, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
         "frac": ach / PEAK_FP8_TFLOPS, "algorithmic_flops_per_launch": fused_flops(M),
         "avg_launch_us": t_fused * 1e6, "launch_spread": stats_us(samples)}
    if clock is not None:
        peak_at = PEAK_FP8_TFLOPS * clock["sclk_ghz"] / clock["peak_sclk_ghz"]
        r.update({"sclk_ghz": clock["sclk_ghz"], "peak_at_measured_clock": peak_at,
                  "frac_at_measured_clock": ach / peak_at})
    return r


def fused_kernel_name(M):
    if M <= 256:
        return "indexer_q_small_kernel (small-batch fused kernel)"
    return ("indexer_q_split_lanes_kernel (split-role fused kernel: GEMM + RoPE + Hadamard + FP4, RoPE rows "
            "from the table's lane-ordered copy)")


def chain_record(c, timing, t_fused, fused_samples, clock):
    M = c.M
    st = timing["step_s"]
    rec = {"tokens": M, "us_per_step": st * 1e6, "tokens_per_s": M / st,
           "forward_median_us": timing["forward_median_us"], "reverse_median_us": timing["reverse_median_us"],
           "step_spread": timing["spread"], "steps_per_replay": timing["steps_per_replay"],
           "fused_kernel": fused_roofline(M, t_fused, fused_samples, clock, fused_kernel_name(M)),
           "chain_minus_fused_us": (st - t_fused) * 1e6}
    if M <= 256:
        # at decode-like sizes the fused kernel streams W: its HBM rate
        gbs = fused_bytes(M) / t_fused / 1e9
        rec["fused_kernel_hbm"] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": fused_bytes(M),
                                   "w_stream_gbs": W_BYTES / t_fused / 1e9}
    return rec


def in_chain_events(c, K):
    """The chain's two kernels with an event pair around each (the events' own
    gaps are in these figures)."""
    import numpy as np
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        c.quant()
        ev[i][1].record()
        c.fused()
        ev[i][2].record()
    torch.cuda.synchronize()
    pct = lambda v: {f"p{q}": float(np.percentile(v, q)) * 1e3 for q in (10, 50, 90)}   # ms -> us
    return {"quant": pct([e[0].elapsed_time(e[1]) for e in ev]), "fused": pct([e[1].elapsed_time(e[2]) for e in ev])}


def eager_chain(c, K):
    """K whole steps launched one after another from Python, events only at
    the two ends."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for _ in range(K):
        c.step()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b) / K
    return {"ms_per_step": ms, "tokens_per_s": c.M / (ms * 1e-3), "wall_us_per_step": wall * 1e6 / K,
            "note": "the same steps launched one after another from Python, events only at the ends"}


# ---------------------------------------------------------------------------
# standalone kernels

def quant_roofline(iqp, S, dev, M, workload, n_sets, reps):
    """The standalone quantizer on X' [M, 7168], rotating buffer sets."""
    import torch
    xq = S.quant_input(workload)
    xs = [xq.to(dev) for _ in range(n_sets)]
    qq = [torch.empty((M, QUANT_K), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    ss = [torch.empty((M, (QUANT_K // 128 + 3) // 4), dtype=torch.int32, device=dev) for _ in range(n_sets)]
    n = max(4 * n_sets, min(100, 400_000_000 // quant_bytes(M, QUANT_K) * n_sets))
    t, samples = graph_launch_time(lambda i: iqp.fp8_quant_1x128_ue8m0(xs[i % n_sets], q=qq[i % n_sets],
                                                                       scales=ss[i % n_sets]), n, reps)
    del xs, qq, ss
    b = quant_bytes(M, QUANT_K)
    return {"kernel": f"fp8_quant_1x128_kernel on [{M},{QUANT_K}] ({n_sets} rotating buffer sets, launches "
                      "back to back from a captured graph)",
            "bound": "hbm", "achieved": b / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": b / t / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": b, "avg_launch_us": t * 1e6,
            "launch_spread": stats_us(samples)}


def copy_ceiling(dev, reps):
    """A plain device copy of 1 GiB (read + write bytes / time): the HBM rate a
    streaming kernel reaches on this machine, as context for the HBM fractions."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t, samples = graph_launch_time(lambda i: dst.copy_(src), 4, reps)
    del src, dst
    return {"what": "torch copy_ of 1 GiB device to device, read + write bytes", "gbs": 2 * (1 << 30) / t / 1e9,
            "frac": 2 * (1 << 30) / t / 1e9 / PEAK_HBM_GBS}


def epilogue_roofline(iqp, S, dev, pos, cs, M, reps):
    import torch
    qin = S.q_bf16_inputs("indexer_q_m4632")
    n_sets = 4
    eq = [qin["q"].to(dev) for _ in range(n_sets)]
    eo = [torch.empty((M, N_HEADS, HEAD_DIM // 2), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    es = [torch.empty((M, N_HEADS, HEAD_DIM // 32), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    t, samples = graph_launch_time(
        lambda i: iqp.indexer_q_rope_hadamard_fp4(eq[i % n_sets], pos, cs, n_heads=N_HEADS, q_fp4=eo[i % n_sets],
                                                  q_scales=es[i % n_sets]), 40, reps)
    del eq, eo, es
    b = epilogue_bytes(M)
    return {"kernel": f"indexer_q_epilogue_kernel (bf16 Q [{M}, 64x128] -> RoPE, Hadamard-128, FP4; {n_sets} "
                      "rotating buffer sets, launches back to back from a captured graph)",
            "bound": "hbm", "achieved": b / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": b / t / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": b, "avg_launch_us": t * 1e6,
            "traffic": measured_traffic("epilogue"), "launch_spread": stats_us(samples)}


def weight_prep_roofline(iqp, dev, reps):
    import numpy as np
    import torch
    wg = np.random.default_rng([100, 1])
    wb = torch.from_numpy((wg.standard_normal((N_HEADS * HEAD_DIM, K_PROJ)) * 0.02).astype(np.float32)).to(
        torch.bfloat16)
    n_sets = 10
    wbs = [wb.to(dev) for _ in range(n_sets)]
    wqs = [torch.empty((N_HEADS * HEAD_DIM, K_PROJ), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    wss = [torch.empty((N_HEADS * HEAD_DIM // 128, K_PROJ // 128), dtype=torch.uint8, device=dev)
           for _ in range(n_sets)]
    t, _ = graph_launch_time(lambda i: iqp.fp8_quant_weight_128x128_ue8m0(
        wbs[i % n_sets], q=wqs[i % n_sets], scales=wss[i % n_sets]), 40, reps)
    del wbs, wqs, wss
    b = N_HEADS * HEAD_DIM * K_PROJ * 3 + (N_HEADS * HEAD_DIM // 128) * (K_PROJ // 128)
    return {"kernel": "fp8_quant_weight_kernel (bf16 W [8192,1536] -> E4M3 + 128x128 UE8M0; off the per-token "
                      "path; 10 rotating sets, graph-replayed)",
            "bound": "hbm", "achieved": b / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": b / t / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": b, "avg_launch_us": t * 1e6}


# ---------------------------------------------------------------------------
# the decode-shaped mix

def decode_mix(iqp, S, dev, w, wsb, reps):
    """256 independent calls, M from {1, 2, 4, 8, 16, 32, 64}: each the
    indexer-Q preparation of X [M, 1536] and the quantization of X' [M, 7168]
    (up to ONE_LAUNCH_WITH_QUANT_MAX_TOKENS tokens, i.e. every call of the
    mix, one launch for both, indexer_q_prep_bf16_with_quant_ws with one
    workspace, whose kernel splits each head's K range from 12 to 64 tokens;
    above, three: the two-call preparation and a standalone quantization).
    Sustained calls/s from one captured graph of the whole mix, hot (one
    weight copy) and cold (call i reads weight copy i % 24: 302 MB, beyond the
    Infinity Cache), and launched back to back from Python (hot, host launch
    cost included); per-call latency = the mean
    call time of its M in a graph of 20 such calls (hot) or of 24 calls over
    the 24 copies (cold), with p50 / p99 over the mix's calls."""
    import numpy as np
    import torch
    max_pos = 131072
    cs = iqp.rope_cos_sin_table(S.ROPE_THETA, max_pos, 64, device=dev)
    ws = iqp.indexer_q_workspace(N_HEADS, device=dev)   # shared by every call: they run in stream order
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

    def three(c, wt):
        iqp.fp8_quant_1x128_ue8m0(c["x"], q=c["a"], scales=c["as"])
        iqp.indexer_q_gemm_rope_fp4(c["a"], c["as"], wt[0], wt[1], c["pos"], cs, n_heads=N_HEADS,
                                    q_fp4=c["q"], q_scales=c["qs"])
        iqp.fp8_quant_1x128_ue8m0(c["xw"], q=c["aw"], scales=c["asw"])

    def one(c, wt):
        # the Q preparation and the quantization of X' in one launch
        iqp.indexer_q_prep_bf16(c["x"], wt[0], wt[1], c["pos"], cs, n_heads=N_HEADS, q_fp4=c["q"],
                                q_scales=c["qs"], quant_beside=c["xw"], quant_beside_out=(c["aw"], c["asw"]),
                                workspace=ws)

    def routed(c, wt):
        (one if c["M"] <= iqp.ONE_LAUNCH_WITH_QUANT_MAX_TOKENS else three)(c, wt)

    hot = (w, wsb)
    n_w = 24
    cold = [(w.clone(), wsb.clone()) for _ in range(n_w)]
    med = lambda v: float(np.median(v))
    t_hot = med(replay_times(capture(lambda _: [routed(c, hot) for c in calls], 1), 1, reps))
    t_cold = med(replay_times(capture(lambda _: [routed(c, cold[i % n_w]) for i, c in enumerate(calls)], 1),
                              1, reps))
    t_one = med(replay_times(capture(lambda _: [one(c, hot) for c in calls], 1), 1, reps))
    # the same mix launched back to back from Python (hot weights): host launch
    # cost included, wall clock between two synchronizations, median of reps
    eager = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for c in calls:
            routed(c, hot)
        torch.cuda.synchronize()
        eager.append(time.perf_counter() - t0)
    t_eager = med(eager)
    print(f"[bench] decode mix: {len(calls) / t_hot:.0f} calls/s hot, {len(calls) / t_cold:.0f} cold (graph "
          f"replay), {len(calls) / t_eager:.0f} launched back to back", file=sys.stderr, flush=True)
    t_three = med(replay_times(capture(lambda _: [three(c, hot) for c in calls], 1), 1, reps))
    lat_hot, lat_cold, lat_k = {}, {}, {}
    for m in sorted({c["M"] for c in calls}):
        c = next(c for c in calls if c["M"] == m)
        lat_hot[m] = med(replay_times(capture(lambda _: [routed(c, hot) for _ in range(20)], 1), 20, 5)) * 1e6
        lat_cold[m] = med(replay_times(capture(lambda _: [routed(c, cold[j]) for j in range(n_w)], 1), n_w, 5)) * 1e6
        if m <= 256:
            lat_k[m] = med(replay_times(capture(lambda _: [iqp.indexer_q_prep_bf16(
                c["x"], w, wsb, c["pos"], cs, n_heads=N_HEADS, q_fp4=c["q"], q_scales=c["qs"], workspace=ws)
                for _ in range(20)], 1), 20, 5)) * 1e6
        print(f"[bench] decode M={m}: {lat_hot[m]:.2f} us hot, {lat_cold[m]:.2f} us cold per call",
              file=sys.stderr, flush=True)
    del cold
    per_hot = np.array([lat_hot[c["M"]] for c in calls])
    per_cold = np.array([lat_cold[c["M"]] for c in calls])
    mix_bytes = float(sum(one_launch_bytes(c["M"]) for c in calls))
    mix_k_s = float(sum(lat_k[c["M"]] for c in calls)) * 1e-6
    return {
        "workload": "decode mix: 256 independent calls, M uniform over {1,2,4,8,16,32,64}; each call X bf16 "
                    "[M,1536] -> FP8 quant -> GEMM + RoPE + Hadamard + FP4 (64 heads) and an FP8 quant of X' "
                    f"[M,7168]: one launch for both up to {iqp.ONE_LAUNCH_WITH_QUANT_MAX_TOKENS} tokens (split over "
                    "K from 12 to 64 tokens, with a workspace), three launches above; positions U[0,131072)",
        "calls_per_s": len(calls) / t_hot, "calls_per_s_cold": len(calls) / t_cold,
        "calls_per_s_eager": len(calls) / t_eager,
        "latency_us_hot": {"p50": float(np.percentile(per_hot, 50)), "p99": float(np.percentile(per_hot, 99))},
        "latency_us_cold": {"p50": float(np.percentile(per_cold, 50)), "p99": float(np.percentile(per_cold, 99))},
        "per_M_call_us_hot": {str(k): v for k, v in lat_hot.items()},
        "per_M_call_us_cold": {str(k): v for k, v in lat_cold.items()},
        "one_launch_path_calls_per_s": len(calls) / t_one, "three_launch_path_calls_per_s": len(calls) / t_three,
        "one_launch_kernel_roofline": {
            "kernel": "indexer_q_small_kernel<bf16 in> (FP8 quant + GEMM + RoPE + Hadamard + FP4, M <= 256; "
                      "split over K from 12 to 64 tokens)",
            "bound": "hbm", "achieved": mix_bytes / mix_k_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": mix_bytes / mix_k_s / 1e9 / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": mix_bytes / len(calls),
            "avg_launch_us": mix_k_s / len(calls) * 1e6},
        "timing": f"median of {reps} replays of one captured graph of the whole mix",
    }


# ---------------------------------------------------------------------------

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
    tflops = fused_flops(M) / us * 1e-6
    return {"what": "torch._scaled_mm (hipBLASLt) e4m3 [M,1536] x [8192,1536]^T, per-tensor scales, bf16 out, "
                    "no epilogue; launches back to back", "avg_launch_us": us, "achieved_tflops": tflops,
            "frac": tflops / PEAK_FP8_TFLOPS}


def cpu_baseline(n_tokens, inp, w_cpu, wsb_cpu):
    """Time the oracle (as it stands) on the first n tokens of the workload:
    its FP8 quantization and its whole fused chain."""
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no cross-GPU step); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if args.replays < 5:
        print("--replays must be at least 5", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp4_quantized_prep_amd as iqp
    import synthetic as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] device {torch.cuda.get_device_name(dev)}; preparing inputs", file=sys.stderr, flush=True)
    w_cpu, wsb_cpu = S.weights()
    w, wsb = w_cpu.to(dev), wsb_cpu.to(dev)
    K, R = args.steps, args.replays
    wl = args.workload

    if wl == "decode":
        rec = decode_mix(iqp, S, dev, w, wsb, R)
        print(json.dumps({"metric": "decode-shaped indexer-Q calls/s (graph replay)", "value": rec["calls_per_s"],
                          "unit": "calls/s", "n_gpus": 1, "steps": 256, "warmup": 1,
                          "ms_per_step": 256 / rec["calls_per_s"] * 1e3, "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "data": "synthetic",
                          "dtype": "fp8-e4m3 (fp32 accumulate), bf16 in, fp4-e2m1 out",
                          "config": {"workload": rec["workload"]}, "decode": rec}), flush=True)
        return

    names = {"all": list(CHAINS), "prefill": [HEADLINE], "prefill128": ["c0_chain_m128"],
             "prefill32k": ["c4_chain_m32768"]}[wl]
    tables = {}
    chains = {n: Chain(iqp, S, dev, w, wsb, tables, n) for n in names}
    for c in chains.values():
        for _ in range(args.warmup):
            c.step()
    torch.cuda.synchronize()

    timing, order = time_chains(chains, K, R)
    records = {}
    for n, c in chains.items():
        t_fused, fs = fused_alone(c, R)
        clock = clock_during(c, iqp) if c.M >= 1024 else None
        records[n] = chain_record(c, timing[n], t_fused, fs, clock)
        if clock is not None:
            records[n]["clock"] = clock
        r = records[n]
        print(f"[bench] {n}: {r['us_per_step']:.1f} us/step (fwd {r['forward_median_us']:.1f}, rev "
              f"{r['reverse_median_us']:.1f}, p10 {r['step_spread']['p10_us']:.1f}, p90 "
              f"{r['step_spread']['p90_us']:.1f}) = {r['tokens_per_s']:.3e} tokens/s; fused "
              f"{t_fused * 1e6:.1f} us = {r['fused_kernel']['achieved']:.0f} TFLOP/s"
              + (f" at {clock['sclk_ghz']:.2f} GHz" if clock else ""), file=sys.stderr, flush=True)

    head = HEADLINE if HEADLINE in chains else names[0]
    hc = chains[head]
    hr = records[head]
    extra = {}
    if wl in ("all", "prefill"):
        extra["in_chain_kernel_us"] = in_chain_events(hc, min(K, 100))
        extra["eager"] = eager_chain(hc, K)
        extra["quant_roofline"] = quant_roofline(iqp, S, dev, 4632, "quant_4632x7168", 5, R)
        extra["quant_roofline"]["traffic"] = measured_traffic("quant")
        print(f"[bench] quantizer [4632,7168]: {extra['quant_roofline']['avg_launch_us']:.1f} us = "
              f"{extra['quant_roofline']['achieved']:.0f} GB/s", file=sys.stderr, flush=True)
        extra["hbm_copy_ceiling"] = copy_ceiling(dev, R)
    if wl in ("all", "prefill32k"):
        q32 = quant_roofline(iqp, S, dev, 32768, "prefill_m32768", 2, R)
        records["c4_chain_m32768"]["quant_32768x7168"] = q32
        print(f"[bench] quantizer [32768,7168]: {q32['avg_launch_us']:.1f} us = {q32['achieved']:.0f} GB/s",
              file=sys.stderr, flush=True)
    if wl == "all":
        records["c3_decode_mix"] = decode_mix(iqp, S, dev, w, wsb, R)
        extra["epilogue_roofline"] = epilogue_roofline(iqp, S, dev, chains[HEADLINE].pos, chains[HEADLINE].cs,
                                                       4632, R)
        extra["weight_prep_roofline"] = weight_prep_roofline(iqp, dev, R)
        if args.vendor_gemm:
            extra["vendor_gemm_context"] = vendor_gemm_context(4632, dev)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline and head == HEADLINE:
        cpu = cpu_baseline(args.cpu_tokens, hc.inp, w_cpu, wsb_cpu)

    roof = dict(hr["fused_kernel"])
    roof["traffic"] = measured_traffic("fused") if head == HEADLINE else None
    roof["mfma_busy_frac_counters"] = measured_mfma_util() if head == HEADLINE else None
    M = hc.M
    result = {
        "metric": "tokens/sec & % roofline: FP8 quant (HBM GB/s) + fused indexer-Q (MFMA util)",
        "value": hr["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": timing[head]["steps_per_replay"],
        "warmup": args.warmup,
        "ms_per_step": hr["us_per_step"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate), bf16 in, fp4-e2m1 out",
        "data": "synthetic",
        "config": {
            "workload": f"indexer-Q chain, {M} tokens: X bf16 [{M},1536] -> FP8 1x128 UE8M0 -> "
                        "Q = A W^T (W [8192,1536] E4M3, 128x128 UE8M0) -> RoPE(64 of 128) -> "
                        f"Hadamard-128 -> FP4 e2m1 [{M},64,64] + UE8M0 [{M},64,4]",
            "tokens": M, "K": K_PROJ, "heads": N_HEADS, "head_dim": HEAD_DIM, "rope_dim": 64,
            "parallelism": "single GPU",
        },
        "timing": {
            "method": f"per config, {timing[head]['steps_per_replay']} steps (4632 tokens; other configs scaled "
                      f"to a similar replay length) captured into one HIP graph, {R} timed replays (event pair "
                      "around each) in forward config order then again in reverse order; the value is the "
                      "average of the two orders' median replays",
            "order_forward": order, "replays_per_order": R,
            "forward_median_us": hr["forward_median_us"], "reverse_median_us": hr["reverse_median_us"],
            **{k: v for k, v in hr["step_spread"].items()},
        },
        "roofline": roof,
        "chain_minus_fused_us": hr["chain_minus_fused_us"],
        "configs": records,
        "cpu_baseline": cpu,
        **extra,
        "runtime": {"hip": torch.version.hip, "torch": torch.__version__,
                    "device": torch.cuda.get_device_name(dev)},
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
