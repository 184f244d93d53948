"""GPU parity: fused indexer-Q kernel (block-scaled FP8 GEMM, RoPE,
Hadamard-128, FP4) against the oracle.

Stage-wise float32 checks go through the diagnostic entry point (same kernel,
float32 output after the GEMM, after RoPE and after the Hadamard rotation);
the FP4 output is checked with the acceptance rule (relative L2 <= 2e-2,
boundary-only flips, at most 0.1 %). Token counts cover the pages' test set
(1, 4, 5, 8, 128), ragged tails, the 4,632-token prefill (sampled tokens) and
a 32,768-token heavy-tailed prefill (sampled tokens)."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C
from oracle import indexer_q as IQ
from oracle import quant_fp8 as QO

from gpu_util import mfma_error_bound, oracle_chain_from_x, weights_for_heads

pytestmark = pytest.mark.gpu

THETA = S.ROPE_THETA


@pytest.fixture(scope="module")
def weights():
    codes, sb = S.weights()
    return codes, sb, codes.cuda(), sb.cuda()


@pytest.fixture(scope="module")
def table(gpu_lib):
    return {mp: gpu_lib.rope_cos_sin_table(THETA, mp, 64) for mp in (4096, 4632, 32768, 131072)}


def device_chain(iqp, x, wd, wsd, pos, cs, n_heads=64, layout="k"):
    a, a_s = iqp.fp8_quant_1x128_ue8m0(x.cuda(), scale_layout=layout)
    q, s = iqp.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pos.cuda(), cs, n_heads=n_heads)
    torch.cuda.synchronize()
    return a, a_s, q.cpu().numpy(), s.cpu().numpy()


def test_rope_table_matches_oracle(gpu_lib, table):
    for mp, t in table.items():
        got = t.cpu().numpy().astype(np.float64)
        rows = np.unique(np.concatenate([np.arange(min(mp, 64)), np.random.default_rng(mp).integers(0, mp, 256), [mp - 1]]))
        want = IQ.rope_cos_sin_table(THETA, mp, 64)[rows]
        tol = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64) + 1e-10
        assert np.all(np.abs(got[rows] - want) <= tol), mp


def test_gemm_rope_hadamard_stages_float32(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128")
    x, pos = inp["x"], inp["positions"]
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    cs = table[4096]
    M = x.shape[0]
    a_sb = QO.unpack_scale_words(ref["a_words"], 12)
    bound = mfma_error_bound(ref["a_codes"], a_sb, codes.numpy(), sb.numpy()) + 2.0 ** -20 * np.abs(ref["q"].reshape(M, -1))
    head_bound = np.linalg.norm(bound.reshape(M, 64, 128), axis=2)
    for stage, key in ((0, "q"), (1, "q_rope"), (2, "z")):
        out = gpu_lib.debug_indexer_q_f32(a, a_s, wd, wsd, pos.cuda(), cs, stage).cpu().numpy()
        want = ref[key].reshape(M, -1)
        err = C.rel_l2(out, want)
        print(f"stage {stage}: rel_l2 {err:.3e}, max |err|/bound {np.max(np.abs(out - want) / bound):.3e}")
        assert err <= 2e-4, (stage, err)
        if stage == 0:
            assert np.all(np.abs(out - want) <= bound), stage
        else:
            # RoPE is a rotation and the normalised Hadamard is orthonormal:
            # the error norm of each head cannot grow past the GEMM's
            d = np.linalg.norm((out - want).reshape(M, 64, 128), axis=2)
            assert np.all(d <= head_bound * (1 + 1e-3) + 1e-6 * np.linalg.norm(ref[key], axis=2)), stage


@pytest.mark.parametrize("M", [1, 4, 5, 8, 16, 128, 300])
def test_fused_chain_small_and_ragged(gpu_lib, weights, table, M):
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"], inp["positions"]
    _, _, q, s = device_chain(gpu_lib, x, wd, wsd, pos, table[4096])
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])
    print(f"M={M}", rep)
    assert rep["ok"], rep


@pytest.mark.parametrize("M", [31, 32, 33, 64, 65, 129, 255, 256, 257])
def test_fused_chain_small_batch_boundaries(gpu_lib, weights, table, M):
    """Token counts at the edges of the small-batch kernel's 32-token column
    tiles (1 to 8 tiles up to 256 tokens) and just past it (257: the
    128-token tile kernel); every token checked."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"], inp["positions"]
    _, _, q, s = device_chain(gpu_lib, x, wd, wsd, pos, table[4096])
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])
    print(f"M={M}", rep)
    assert rep["ok"], rep


def test_fused_chain_mn_major_scales(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=77)
    x, pos = inp["x"], inp["positions"]
    _, _, q, s = device_chain(gpu_lib, x, wd, wsd, pos, table[4096], layout="mn")
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    assert C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])["ok"]


@pytest.mark.parametrize("H", [1, 3, 8])
def test_fused_chain_other_head_counts(gpu_lib, table, H):
    codes, sb = weights_for_heads(H)
    inp = S.indexer_q_inputs("indexer_q_m128", M=70)
    x, pos = inp["x"], inp["positions"]
    _, _, q, s = device_chain(gpu_lib, x, codes.cuda(), sb.cuda(), pos, table[4096], n_heads=H)
    ref = oracle_chain_from_x(x, codes, sb, pos, H)
    assert C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])["ok"]


@pytest.mark.parametrize("K", [1024, 2048])
def test_fused_chain_other_k(gpu_lib, table, K):
    """K other than 1536 runs the general (non-pipelined) fused kernel."""
    H, M = 4, 70
    codes, sb = S.weights(N=H * 128, K=K, seed=101)
    g = S.rng("indexer_q_m128", 900 + K)
    x = S.activations_outlier(g, M, K)
    pos = S.positions_uniform(g, M, 4096)
    _, _, q, s = device_chain(gpu_lib, x, codes.cuda(), sb.cuda(), pos, table[4096], n_heads=H)
    ref = oracle_chain_from_x(x, codes, sb, pos, H)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])
    print(f"K={K}", rep)
    assert rep["ok"], rep


@pytest.mark.parametrize("M", [1157, 2309])
def test_fused_chain_uneven_tile_chunks(gpu_lib, weights, table, M):
    """Token counts whose 128-token tiles split unevenly over the 8 chunks of
    each of the 32 head pairs (1 or 2 tiles per chunk at 1157, 2 or 3 at
    2309), with a ragged last tile; every token checked."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"], inp["positions"]
    _, _, q, s = device_chain(gpu_lib, x, wd, wsd, pos, table[4096])
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])
    print(f"M={M}", rep)
    assert rep["ok"], rep


@pytest.mark.parametrize("M,H,max_pos", [(256, 64, 4096), (257, 64, 4096), (383, 3, 4096), (1023, 64, 4096),
                                         (1024, 64, 4096), (1300, 3, 131072), (1100, 1, 4096),
                                         (2100, 8, 131072), (1500, 64, 131072)])
def test_fused_chain_split_build(gpu_lib, table, M, H, max_pos):
    """Token counts on both sides of the switch from the small-batch kernel
    to the split-role build of the pipelined kernel (257 tokens: one tile a
    workgroup, a partial second tile), odd and single head counts (a head
    pair with no second head), positions up to 131071; every token
    checked."""
    codes, sb = weights_for_heads(H)
    g = S.rng("indexer_q_m128", 1200 + M)
    x = S.activations_outlier(g, M, 1536)
    pos = S.positions_uniform(g, M, max_pos)
    pos[0], pos[-1] = 0, max_pos - 1
    _, _, q, s = device_chain(gpu_lib, x, codes.cuda(), sb.cuda(), pos, table[max_pos], n_heads=H)
    ref = oracle_chain_from_x(x, codes, sb, pos, H)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])
    print(f"M={M} H={H}", rep)
    assert rep["ok"], rep


def _sampled_check(iqp, weights, x, pos, cs, n_sample, seed):
    codes, sb, wd, wsd = weights
    _, _, q, s = device_chain(iqp, x, wd, wsd, pos, cs)
    M = x.shape[0]
    rows = np.random.default_rng(seed).choice(M, n_sample, replace=False)
    rows = np.unique(np.concatenate([rows, [0, M - 1]]))
    ref = oracle_chain_from_x(x[rows], codes, sb, pos[rows], 64)
    rep = C.check_fp4(q[rows], s[rows], ref["z"], ref["q_fp4"], ref["q_scales"])
    print(f"M={M} sampled", rep)
    assert rep["ok"], rep


def test_fused_chain_m4632_sampled(gpu_lib, weights, table):
    inp = S.indexer_q_inputs("indexer_q_m4632")
    _sampled_check(gpu_lib, weights, inp["x"], inp["positions"], table[4632], 384, 1)


def test_fused_chain_m32768_student_t_sampled(gpu_lib, weights, table):
    inp = S.indexer_q_inputs("prefill_m32768")
    _sampled_check(gpu_lib, weights, inp["x"], inp["positions"], table[32768], 384, 2)


def test_decode_calls_large_positions(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    for call in S.decode_calls(12):
        x, pos = call["x"], call["positions"]
        _, _, q, s = device_chain(gpu_lib, x, wd, wsd, pos, table[131072])
        ref = oracle_chain_from_x(x, codes, sb, pos, 64)
        rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])
        assert rep["ok"], (x.shape, rep)


def test_every_output_byte_written_and_no_overrun(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=37)
    x, pos = inp["x"].cuda(), inp["positions"].cuda()
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x)
    M, H = 37, 64
    results = []
    for fill in (0x00, 0xFF):
        qbuf = torch.full((M * H * 64 + 256,), fill, dtype=torch.uint8, device="cuda")
        sbuf = torch.full((M * H * 4 + 256,), fill, dtype=torch.uint8, device="cuda")
        q = qbuf[128:128 + M * H * 64].view(M, H, 64)
        s = sbuf[128:128 + M * H * 4].view(M, H, 4)
        gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pos, table[4096], q_fp4=q, q_scales=s)
        qh, sh = qbuf.cpu().numpy(), sbuf.cpu().numpy()
        for buf, n in ((qh, M * H * 64), (sh, M * H * 4)):
            assert np.all(buf[:128] == fill) and np.all(buf[128 + n:] == fill)
        results.append((q.cpu(), s.cpu()))
    assert torch.equal(results[0][0], results[1][0]) and torch.equal(results[0][1], results[1][1])


@pytest.mark.parametrize("M", [8, 128])
def test_graph_capture_replays_match_eager(gpu_lib, weights, table, M):
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"].cuda(), inp["positions"].cuda()
    cs = table[4096]
    q_e, s_e = gpu_lib.indexer_q_prep(x, wd, wsd, pos, cs)
    q_e, s_e = q_e.clone(), s_e.clone()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        gpu_lib.indexer_q_prep(x, wd, wsd, pos, cs)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q_g, s_g = gpu_lib.indexer_q_prep(x, wd, wsd, pos, cs)
    for _ in range(5):
        q_g.zero_()
        s_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q_g, q_e) and torch.equal(s_g, s_e)
        # eager work between replays
        gpu_lib.indexer_q_prep(x, wd, wsd, pos, cs)
        torch.cuda.synchronize()


def test_unsupported_shapes_raise(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    x = S.indexer_q_inputs("indexer_q_m128", M=4)["x"].cuda()
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x)
    pos = torch.zeros(4, dtype=torch.int64, device="cuda")
    with pytest.raises(gpu_lib.IqpError) as e:
        gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, wd[:8192], wsd, pos, table[4096][:, :32].contiguous(),
                                        rope_dim=32)
    assert e.value.status == gpu_lib.IQP_ERR_UNSUPPORTED


# ---------------------------------------------------------------- convention variants

FUSED_VARIANTS = [("interleaved", "ceil"), ("half_split", "ocp_floor"), ("interleaved", "ocp_floor")]


def device_chain_variant(iqp, x, wd, wsd, pos, cs, n_heads, layout, rule):
    a, a_s = iqp.fp8_quant_1x128_ue8m0(x.cuda())
    q, s = iqp.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pos.cuda(), cs, n_heads=n_heads, rope_layout=layout,
                                       scale_rule=rule)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("layout,rule", FUSED_VARIANTS)
@pytest.mark.parametrize("M", [1, 5, 33, 128, 256, 300, 1157])
def test_fused_chain_variants(gpu_lib, weights, table, layout, rule, M):
    """The flags call (indexer_q_gemm_rope_fp4_ex) against the oracle's chain
    with the same conventions; every token checked. Up to 256 tokens the
    small-batch kernel's variant build runs, above it the pipelined kernel's
    (1157: uneven tile chunks)."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"], inp["positions"]
    print(f"[variant] M={M} {layout} {rule}", flush=True)
    q, s = device_chain_variant(gpu_lib, x, wd, wsd, pos, table[4096], 64, layout, rule)
    ref = oracle_chain_from_x(x, codes, sb, pos, 64, layout, rule)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"], scale_rule=rule)
    print(rep)
    assert rep["ok"], rep
    if M == 128:
        assert rep["rel_l2"] < 2e-2


@pytest.mark.parametrize("layout,rule", FUSED_VARIANTS)
def test_fused_chain_variants_other_k_and_heads(gpu_lib, table, layout, rule):
    H, M, K = 3, 70, 1024
    codes, sb = S.weights(N=H * 128, K=K, seed=101)
    g = S.rng("indexer_q_m128", 900 + K)
    x = S.activations_outlier(g, M, K)
    pos = S.positions_uniform(g, M, 4096)
    q, s = device_chain_variant(gpu_lib, x, codes.cuda(), sb.cuda(), pos, table[4096], H, layout, rule)
    ref = oracle_chain_from_x(x, codes, sb, pos, H, layout, rule)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"], scale_rule=rule)
    assert rep["ok"], rep


@pytest.mark.parametrize("layout,rule", FUSED_VARIANTS)
def test_fused_variant_split_build_three_heads(gpu_lib, table, layout, rule):
    """The split-role variant builds with 3 heads (the second pair without
    its second head) and 1100 tokens (uneven tile chunks), every token."""
    H, M, K = 3, 1100, 1536
    codes, sb = S.weights(N=H * 128, K=K, seed=106)
    g = S.rng("indexer_q_m4632", 962)
    x = S.activations_outlier(g, M, K)
    pos = S.positions_uniform(g, M, 32768)
    print(f"[variant] M={M} H={H} {layout} {rule} (split-role build)", flush=True)
    q, s = device_chain_variant(gpu_lib, x, codes.cuda(), sb.cuda(), pos, table[32768], H, layout, rule)
    ref = oracle_chain_from_x(x, codes, sb, pos, H, layout, rule)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"], scale_rule=rule)
    assert rep["ok"], rep


@pytest.mark.parametrize("layout", ["interleaved", "half_split"])
def test_fused_chain_variant_m4632_sampled(gpu_lib, weights, table, layout):
    """4632 tokens with the floor rule (the split-role variant builds)."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m4632")
    x, pos = inp["x"], inp["positions"]
    print(f"[variant] M=4632 {layout} ocp_floor", flush=True)
    q, s = device_chain_variant(gpu_lib, x, wd, wsd, pos, table[4632], 64, layout, "ocp_floor")
    rows = np.unique(np.concatenate([np.arange(8), np.random.default_rng(4634).integers(0, 4632, 120),
                                     np.arange(4632 - 8, 4632)]))
    ref = oracle_chain_from_x(x[rows], codes, sb, pos[rows], 64, layout, "ocp_floor")
    rep = C.check_fp4(q[rows], s[rows], ref["z"], ref["q_fp4"], ref["q_scales"], scale_rule="ocp_floor")
    assert rep["ok"], rep


@pytest.mark.parametrize("layout,rule", FUSED_VARIANTS)
@pytest.mark.parametrize("M", [1024, 2048])
def test_fused_variant_split_build_every_token(gpu_lib, weights, table, layout, rule, M):
    """Above 256 tokens the flags call runs the split-role variant builds
    (indexer_q_split_v1..3.hip): every token against the oracle, at 8 and
    16 tiles a head pair; scattered positions, so that
    each lane's RoPE rows come from all over the table."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m4632")
    x = inp["x"][:M]
    pos = S.positions_uniform(S.rng("indexer_q_m4632", 77 + M), M, 32768)
    print(f"[variant] M={M} {layout} {rule} (split-role build)", flush=True)
    q, s = device_chain_variant(gpu_lib, x, wd, wsd, pos, table[32768], 64, layout, rule)
    ref = oracle_chain_from_x(x, codes, sb, pos, 64, layout, rule)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"], scale_rule=rule)
    print(rep)
    assert rep["ok"], rep


def test_fused_ex_flags_zero_is_the_base_call(gpu_lib, weights, table):
    """flags = 0 through indexer_q_gemm_rope_fp4_ex writes the base call's
    bytes (every output byte, over guard-filled buffers)."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=40)
    x, pos = inp["x"], inp["positions"]
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    pd = pos.cuda()
    q0, s0 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pd, table[4096], n_heads=64)
    _, args = gpu_lib._indexer_q_common(a, a_s, wd, wsd, pd, table[4096], 64, 128, 64)
    q1 = torch.full_like(q0, 0x5A)
    s1 = torch.full_like(s0, 0xA5)
    st = gpu_lib._lib.indexer_q_gemm_rope_fp4_ex(*args, q1.data_ptr(), s1.data_ptr(), 0,
                                                 torch.cuda.current_stream().cuda_stream)
    assert st == gpu_lib.IQP_OK
    torch.cuda.synchronize()
    assert torch.equal(q0.cpu(), q1.cpu()) and torch.equal(s0.cpu(), s1.cpu())


# ---------------------------------------------------------------- maximum K, zero rows


def test_fused_chain_maximum_k(gpu_lib, table):
    """K = 32768, the largest K the fused call takes (256 K blocks, the general
    kernel), 40 tokens x 2 heads; every token checked."""
    H, M, K = 2, 40, 32768
    codes, sb = S.weights(N=H * 128, K=K, seed=102)
    g = S.rng("indexer_q_m128", 950)
    x = S.activations_outlier(g, M, K)
    pos = S.positions_uniform(g, M, 4096)
    print(f"[max K] M={M} K={K} H={H}", flush=True)
    _, _, q, s = device_chain(gpu_lib, x, codes.cuda(), sb.cuda(), pos, table[4096], n_heads=H)
    ref = oracle_chain_from_x(x, codes, sb, pos, H)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])
    print(rep)
    assert rep["ok"], rep


@pytest.mark.parametrize("M", [5, 300])
def test_fused_chain_zero_token_rows(gpu_lib, weights, table, M):
    """All-zero activation rows (the small-batch kernel at 5 tokens, the
    pipelined kernel at 300): their Q is exactly zero, so every FP4 block of
    theirs takes the floor exponent -15 (byte 112) and every code is a zero
    (+0 or -0: RoPE with a negative cosine turns 0 into -0); the other rows
    are unaffected."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"].clone(), inp["positions"]
    zero_rows = [0, M // 2, M - 1]
    x[zero_rows] = 0
    _, _, q, s = device_chain(gpu_lib, x, wd, wsd, pos, table[4096])
    assert np.all(s[zero_rows] == 112) and np.all((q[zero_rows] & 0x77) == 0)
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    rep = C.check_fp4(q, s, ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep


# ---------------------------------------------------------------- per-row (1x128) weight scales


def row_scale_weights(H, K, seed):
    """E4M3 weight codes [H*128, K] with one UE8M0 byte per row and K block:
    the synthetic tile bytes, each row's moved by -1, 0 or +1 per block."""
    codes, sb = S.weights(N=H * 128, K=K, seed=seed)
    g = np.random.default_rng([seed, 7])
    rows = np.repeat(sb.numpy().astype(np.int64), 128, axis=0) + g.integers(-1, 2, size=(H * 128, K // 128))
    return codes, torch.from_numpy(rows.astype(np.uint8))


@pytest.mark.parametrize("M,H,K", [(1, 64, 1536), (5, 64, 1536), (128, 64, 1536), (256, 64, 1536),
                                   (300, 64, 1536), (1157, 64, 1536), (2048, 64, 1536), (300, 3, 1536),
                                   (1100, 3, 1536), (70, 3, 1024)])
def test_fused_chain_row_weight_scales(gpu_lib, table, M, H, K):
    """At K = 1536 the small-batch kernel's per-row build runs up to 256
    tokens and the pipelined kernel's one-role build above, also where other
    calls take the split-role builds (1157: uneven tile chunks; 3 heads: a
    pair without its second head); the general kernel at K = 1024."""
    codes, wsr = row_scale_weights(H, K, 103)
    if K == 1536:
        inp = S.indexer_q_inputs("indexer_q_m128", M=M)
        x, pos = inp["x"], inp["positions"]
    else:
        g = S.rng("indexer_q_m128", 960)
        x = S.activations_outlier(g, M, K)
        pos = S.positions_uniform(g, M, 4096)
    print(f"[row scales] M={M} H={H} K={K}", flush=True)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    q, s = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), wsr.cuda(), pos.cuda(), table[4096], n_heads=H,
                                           w_scale_layout="row_1x128")
    torch.cuda.synchronize()
    ref = oracle_chain_from_x(x, codes, wsr, pos, H)
    rep = C.check_fp4(q.cpu().numpy(), s.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    print(rep)
    assert rep["ok"], rep


@pytest.mark.parametrize("K,M", [(1024, 90), (1536, 90), (1536, 600)])
def test_row_weight_scales_equal_to_tile_scales_give_the_same_bytes(gpu_lib, table, K, M):
    """Per-row bytes that repeat each tile's byte over its 128 rows: the same
    output bytes as the per-tile call (the general kernel at K = 1024, the
    small-batch kernel's builds at 90 tokens and the pipelined kernel's at 600
    when K = 1536), for the default and the interleaved / floor-rule
    conventions."""
    H = 4
    codes, sb = S.weights(N=H * 128, K=K, seed=104)
    rows = torch.from_numpy(np.repeat(sb.numpy(), 128, axis=0).copy())
    g = S.rng("indexer_q_m128", 961)
    x = S.activations_outlier(g, M, K)
    pos = S.positions_uniform(g, M, 4096).cuda()
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    for layout, rule in (("half_split", "ceil"), ("interleaved", "ocp_floor")):
        q0, s0 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), sb.cuda(), pos, table[4096], n_heads=H,
                                                 rope_layout=layout, scale_rule=rule)
        q1, s1 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), rows.cuda(), pos, table[4096], n_heads=H,
                                                 rope_layout=layout, scale_rule=rule, w_scale_layout="row_1x128")
        torch.cuda.synchronize()
        assert torch.equal(q0.cpu(), q1.cpu()) and torch.equal(s0.cpu(), s1.cpu()), (layout, rule)


@pytest.mark.parametrize("M", [70, 300, 1100])
def test_row_weight_scales_with_variants(gpu_lib, table, M):
    H, K = 3, 1536
    codes, wsr = row_scale_weights(H, K, 105)
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"], inp["positions"]
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    q, s = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), wsr.cuda(), pos.cuda(), table[4096], n_heads=H,
                                           rope_layout="interleaved", scale_rule="ocp_floor",
                                           w_scale_layout="row_1x128")
    torch.cuda.synchronize()
    ref = oracle_chain_from_x(x, codes, wsr, pos, H, "interleaved", "ocp_floor")
    rep = C.check_fp4(q.cpu().numpy(), s.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"],
                      scale_rule="ocp_floor")
    assert rep["ok"], rep
