"""GPU parity: the one-launch decode path (bf16 X in; FP8 quantization,
block-scaled FP8 projection, RoPE, Hadamard-128, FP4 in one kernel).

Its FP4 output must pass the oracle's acceptance rule, and it must be byte
for byte the output of the two-call path (fp8_quant_1x128_ue8m0, then
indexer_q_gemm_rope_fp4), since it quantizes with the same arithmetic and
runs the same MFMA and epilogue code. Cases: every 32-token tile boundary up
to 256 tokens, the decode mix's large positions, other head counts, strided
rows, quantization edge blocks (x1e3, x1e-6, all-zero, bf16 subnormals), graph
replay, guard bytes and the shapes it declines."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C

from gpu_util import oracle_chain_from_x, weights_for_heads

pytestmark = pytest.mark.gpu

THETA = S.ROPE_THETA


@pytest.fixture(scope="module")
def weights():
    codes, sb = S.weights()
    return codes, sb, codes.cuda(), sb.cuda()


@pytest.fixture(scope="module")
def table(gpu_lib):
    return {mp: gpu_lib.rope_cos_sin_table(THETA, mp, 64) for mp in (4096, 131072)}


def two_call(iqp, x, wd, wsd, pos, cs, n_heads=64):
    a, a_s = iqp.fp8_quant_1x128_ue8m0(x)
    return iqp.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pos, cs, n_heads=n_heads)


def check(iqp, x, codes, sb, wd, wsd, pos, cs, n_heads=64, x_dev=None):
    print(f"[prep_bf16] M={x.shape[0]} H={n_heads}", flush=True)
    xd = x.cuda() if x_dev is None else x_dev
    q1, s1 = iqp.indexer_q_prep_bf16(xd, wd, wsd, pos.cuda(), cs, n_heads=n_heads)
    q2, s2 = two_call(iqp, xd, wd, wsd, pos.cuda(), cs, n_heads=n_heads)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2), "one launch differs from the two-call path"
    ref = oracle_chain_from_x(x, codes, sb, pos, n_heads)
    rep = C.check_fp4(q1.cpu().numpy(), s1.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep


@pytest.mark.parametrize("M", [1, 2, 4, 5, 8, 16, 31, 32, 33, 64, 65, 128, 200, 255, 256])
def test_one_launch_token_counts(gpu_lib, weights, table, M):
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    check(gpu_lib, inp["x"], codes, sb, wd, wsd, inp["positions"], table[4096])


def test_one_launch_decode_calls(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    for call in S.decode_calls(12):
        check(gpu_lib, call["x"], codes, sb, wd, wsd, call["positions"], table[131072])


@pytest.mark.parametrize("H", [1, 3])
def test_one_launch_other_head_counts(gpu_lib, table, H):
    codes, sb = weights_for_heads(H)
    inp = S.indexer_q_inputs("indexer_q_m128", M=37)
    check(gpu_lib, inp["x"], codes, sb, codes.cuda(), sb.cuda(), inp["positions"], table[4096], n_heads=H)


def test_one_launch_strided_rows(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=40)
    wide = torch.zeros((40, 1536 + 64), dtype=torch.bfloat16)
    wide[:, 32:32 + 1536] = inp["x"]
    view = wide.cuda()[:, 32:32 + 1536]
    assert view.stride(0) == 1600
    check(gpu_lib, inp["x"], codes, sb, wd, wsd, inp["positions"], table[4096], x_dev=view)


def test_one_launch_quantization_edge_blocks(gpu_lib, weights, table):
    """x1e3 and x1e-6 blocks (the tiny-scale floor), an all-zero row and a row
    of bf16 subnormals: the in-kernel quantization must give the standalone
    quantizer's bytes, so the outputs stay identical."""
    codes, sb, wd, wsd = weights
    x = S.quant_input("quant_4632x7168", M=48, K=1536).clone()
    x[5] = 0
    x[9] = torch.from_numpy((np.arange(1536, dtype=np.uint32) % 127 + 1).astype(np.int16)).view(torch.bfloat16)
    pos = S.indexer_q_inputs("indexer_q_m128", M=48)["positions"]
    check(gpu_lib, x, codes, sb, wd, wsd, pos, table[4096])


def test_one_launch_graph_replays_match_eager(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=24)
    x, pos = inp["x"].cuda(), inp["positions"].cuda()
    cs = table[4096]
    q_e, s_e = gpu_lib.indexer_q_prep_bf16(x, wd, wsd, pos, cs)
    q_e, s_e = q_e.clone(), s_e.clone()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        gpu_lib.indexer_q_prep_bf16(x, wd, wsd, pos, cs)
    torch.cuda.current_stream().wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q_g, s_g = gpu_lib.indexer_q_prep_bf16(x, wd, wsd, pos, cs)
    for _ in range(4):
        q_g.zero_()
        s_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q_g, q_e) and torch.equal(s_g, s_e)
        gpu_lib.indexer_q_prep_bf16(x, wd, wsd, pos, cs)
        torch.cuda.synchronize()


def test_one_launch_no_write_outside_outputs(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    M, H = 7, 64
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    n_codes, n_sc = M * H * 64, M * H * 4
    cbuf = torch.full((n_codes + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((n_sc + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    q = cbuf[32:32 + n_codes].view(M, H, 64)
    s = sbuf[32:32 + n_sc].view(M, H, 4)
    gpu_lib.indexer_q_prep_bf16(inp["x"].cuda(), wd, wsd, inp["positions"].cuda(), table[4096], q_fp4=q, q_scales=s)
    ch, sh = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(ch[:32] == 0x5A) and np.all(ch[32 + n_codes:] == 0x5A)
    assert np.all(sh[:32] == 0xA5) and np.all(sh[32 + n_sc:] == 0xA5)
    q2, s2 = two_call(gpu_lib, inp["x"].cuda(), wd, wsd, inp["positions"].cuda(), table[4096])
    assert torch.equal(q, q2) and torch.equal(s, s2)


def test_one_launch_declines_large_batches_and_other_k(gpu_lib, weights, table):
    codes, sb, wd, wsd = weights
    x = S.indexer_q_inputs("indexer_q_m128", M=257)["x"].cuda()
    pos = torch.zeros(257, dtype=torch.int64, device="cuda")
    with pytest.raises(gpu_lib.IqpError) as e:
        gpu_lib.indexer_q_prep_bf16(x, wd, wsd, pos, table[4096])
    assert e.value.status == gpu_lib.IQP_ERR_UNSUPPORTED
    codes2, sb2 = S.weights(K=1024)
    x2 = torch.zeros((4, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.IqpError) as e:
        gpu_lib.indexer_q_prep_bf16(x2, codes2.cuda(), sb2.cuda(), pos[:4], table[4096])
    assert e.value.status == gpu_lib.IQP_ERR_UNSUPPORTED


# ---------------------------------------------------------------- convention flags (indexer_q_prep_bf16_ex)

FLAG_CASES = [("interleaved", "ceil", "tile_128x128"), ("half_split", "ocp_floor", "tile_128x128"),
              ("interleaved", "ocp_floor", "tile_128x128"), ("half_split", "ceil", "row_1x128"),
              ("interleaved", "ocp_floor", "row_1x128")]


@pytest.mark.parametrize("layout,rule,wlayout", FLAG_CASES)
@pytest.mark.parametrize("M", [1, 16, 33, 256])
def test_one_launch_flags_match_two_calls_and_oracle(gpu_lib, weights, table, layout, rule, wlayout, M):
    """With convention flags the one-launch call is byte for byte the two-call
    path with the same flags, and passes the oracle's rule for them."""
    codes, sb, wd, wsd = weights
    if wlayout == "row_1x128":
        g = np.random.default_rng([103, 8])
        rows = np.repeat(sb.numpy().astype(np.int64), 128, axis=0) + g.integers(-1, 2, size=(64 * 128, 12))
        sb = torch.from_numpy(rows.astype(np.uint8))
        wsd = sb.cuda()
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"], inp["positions"]
    print(f"[prep_bf16 flags] M={M} {layout} {rule} {wlayout}", flush=True)
    kw = dict(rope_layout=layout, scale_rule=rule, w_scale_layout=wlayout)
    q1, s1 = gpu_lib.indexer_q_prep_bf16(x.cuda(), wd, wsd, pos.cuda(), table[4096], **kw)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    q2, s2 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pos.cuda(), table[4096], **kw)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2), "one launch differs from the two-call path"
    ref = oracle_chain_from_x(x, codes, sb, pos, 64, layout, rule)
    rep = C.check_fp4(q1.cpu().numpy(), s1.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"], scale_rule=rule)
    assert rep["ok"], rep


@pytest.mark.parametrize("M", [8, 300])
def test_routing_helper_passes_the_flags(gpu_lib, weights, table, M):
    """indexer_q_prep (one launch at 8 tokens, two calls at 300) with flags
    gives the bytes of the direct two-call path with the same flags."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"].cuda(), inp["positions"].cuda()
    kw = dict(rope_layout="interleaved", scale_rule="ocp_floor")
    q1, s1 = gpu_lib.indexer_q_prep(x, wd, wsd, pos, table[4096], **kw)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x)
    q2, s2 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pos, table[4096], **kw)
    q0, _ = gpu_lib.indexer_q_prep(x, wd, wsd, pos, table[4096])
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    assert not torch.equal(q1, q0)


@pytest.mark.parametrize("M,M2,K2,layout", [(1, 1, 7168, "k"), (5, 7, 640, "k"), (16, 64, 7168, "mn"),
                                            (100, 3, 7168, "k"), (256, 256, 7168, "k"), (0, 9, 7168, "k")])
def test_one_launch_with_quant_beside_matches_separate_calls(gpu_lib, weights, table, M, M2, K2, layout):
    """indexer_q_prep_bf16_with_quant: the Q preparation and the quantization
    of an independent matrix in one launch give byte for byte the outputs of
    the two separate calls (a ragged last word at K2 = 640, MN-major words,
    no tokens for the projection)."""
    codes, sb, wd, wsd = weights
    inp = S.indexer_q_inputs("indexer_q_m128", M=max(M, 1))
    x = inp["x"][:M].cuda()
    pos = inp["positions"][:M].cuda()
    g = S.rng("decode_mix", 4000 + M2 + K2)
    x2 = S.activations_outlier(g, M2, K2).cuda()
    print(f"[prep_bf16 + quant] M={M} M2={M2} K2={K2} {layout}", flush=True)
    q, s, q2, s2 = gpu_lib.indexer_q_prep_bf16(x, wd, wsd, pos, table[4096], quant_beside=x2,
                                                quant_beside_layout=layout)
    r2, rs2 = gpu_lib.fp8_quant_1x128_ue8m0(x2, scale_layout=layout)
    if M:
        r, rs = gpu_lib.indexer_q_prep_bf16(x, wd, wsd, pos, table[4096])
    torch.cuda.synchronize()
    assert torch.equal(q2, r2) and torch.equal(s2, rs2), "the quantization beside differs"
    if M:
        assert torch.equal(q, r) and torch.equal(s, rs), "the Q preparation differs"
