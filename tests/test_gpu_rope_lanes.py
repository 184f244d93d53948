"""GPU: the RoPE table's lane-ordered copy (iqp_rope_table_lanes) and the
fused call that reads it (indexer_q_gemm_rope_fp4_lanes).

The copy is a rearrangement of the table, so it is checked bit for bit
against that rearrangement written out here from its definition in
include/iqprep.h. The fused call must give the bytes of the call that reads
the table itself, whatever the positions: consecutive (aligned to the
32-position blocks or not), packed sequences restarting at 0, scattered, and
a token count of the small-batch kernel (where the table is read). One
ragged prefill is also checked against the oracle, every token."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C

from gpu_util import oracle_chain_from_x, weights_for_heads

pytestmark = pytest.mark.gpu


def lanes_definition(cs: np.ndarray) -> np.ndarray:
    """Element 2048 b + 256 L + 4 (2 r + h) + e = cs[32 b + r, 32 (L % 2) +
    8 (L // 2) + 4 h + e], zero past the table's last row."""
    mp = cs.shape[0]
    nb = (mp + 31) // 32
    rows = np.zeros((nb * 32, 64), np.float32)
    rows[:mp] = cs
    rows = rows.reshape(nb, 32, 64)
    out = np.zeros((nb, 8, 32, 2, 4), np.float32)
    for L in range(8):
        for h in range(2):
            c0 = 32 * (L % 2) + 8 * (L // 2) + 4 * h
            out[:, L, :, h, :] = rows[:, :, c0:c0 + 4]
    return out.reshape(-1)


@pytest.mark.parametrize("max_pos", [1, 31, 1000, 4100, 4632, 32768])
def test_lane_table_layout(gpu_lib, max_pos):
    g = np.random.default_rng(max_pos)
    cs = torch.from_numpy(g.standard_normal((max_pos, 64)).astype(np.float32)).cuda()
    got = gpu_lib.rope_table_lanes(cs)
    torch.cuda.synchronize()
    assert tuple(got.shape) == (gpu_lib.rope_table_lanes_size(max_pos),)
    want = lanes_definition(cs.cpu().numpy())
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


def _positions(kind: str, M: int, max_pos: int, seed: int) -> torch.Tensor:
    g = np.random.default_rng(seed)
    if kind == "consecutive":
        p = np.arange(M)
    elif kind == "offset":           # a run that starts inside a 32-position block
        p = 5 + np.arange(M)
    elif kind == "table_end":        # a run ending at the last row of a table whose size is not a multiple of 32
        p = max_pos - M + np.arange(M)
    elif kind == "packed":           # sequences of unequal length packed into one batch
        cuts = np.sort(g.choice(np.arange(1, M), 3, replace=False))
        p = np.concatenate([np.arange(n) for n in np.diff(np.concatenate([[0], cuts, [M]]))])
    elif kind == "scattered":
        p = g.integers(0, max_pos, M)
    else:
        raise ValueError(kind)
    assert p.min() >= 0 and p.max() < max_pos
    return torch.from_numpy(p.astype(np.int64))


CASES = [
    # M, heads, table rows, positions
    (4632, 64, 32768, "consecutive"),
    (1061, 64, 32768, "offset"),
    (1100, 64, 4100, "table_end"),
    (3000, 64, 32768, "packed"),
    (2048, 64, 32768, "scattered"),
    (1300, 3, 4096, "offset"),
    (500, 64, 4096, "consecutive"),
    (200, 64, 4096, "consecutive"),      # the small-batch kernel: the table is read
]


@pytest.mark.parametrize("M,H,max_pos,kind", CASES)
def test_fused_lanes_bytes_equal_table_path(gpu_lib, M, H, max_pos, kind):
    codes, sb = weights_for_heads(H)
    wd, wsd = codes.cuda(), sb.cuda()
    g = S.rng("indexer_q_m128", 3100 + M)
    x = S.activations_outlier(g, M, 1536)
    pos = _positions(kind, M, max_pos, M).cuda()
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, max_pos, 64)
    lanes = gpu_lib.rope_table_lanes(cs)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    q0, s0 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pos, cs, n_heads=H)
    q1, s1 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pos, cs, n_heads=H, cos_sin_lanes=lanes)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1) and torch.equal(s0, s1), (M, H, kind)


def test_fused_lanes_m32768_bytes_equal_table_path(gpu_lib):
    inp = S.indexer_q_inputs("prefill_m32768")
    codes, sb = S.weights()
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, inp["max_pos"], 64)
    lanes = gpu_lib.rope_table_lanes(cs)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(inp["x"].cuda())
    pos = inp["positions"].cuda()
    q0, s0 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), sb.cuda(), pos, cs)
    q1, s1 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), sb.cuda(), pos, cs, cos_sin_lanes=lanes)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1) and torch.equal(s0, s1)


def test_fused_lanes_against_oracle(gpu_lib):
    """A ragged prefill whose runs start inside the 32-position blocks:
    the lane-ordered path against the oracle, every token."""
    M, H, max_pos = 1061, 64, 4096
    codes, sb = weights_for_heads(H)
    g = S.rng("indexer_q_m128", 3300)
    x = S.activations_outlier(g, M, 1536)
    pos = _positions("offset", M, max_pos, 7)
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, max_pos, 64)
    lanes = gpu_lib.rope_table_lanes(cs)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    q, s = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), sb.cuda(), pos.cuda(), cs, n_heads=H,
                                           cos_sin_lanes=lanes)
    torch.cuda.synchronize()
    ref = oracle_chain_from_x(x, codes, sb, pos, H)
    rep = C.check_fp4(q.cpu().numpy(), s.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    print(rep)
    assert rep["ok"], rep


def test_lane_table_binding_checks(gpu_lib):
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, 64, 64)
    with pytest.raises(ValueError):
        gpu_lib.rope_table_lanes(cs, out=torch.empty(10, dtype=torch.float32, device="cuda"))
    codes, sb = weights_for_heads(2)
    x = torch.zeros((4, 1536), dtype=torch.bfloat16)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    pos = torch.zeros(4, dtype=torch.int64, device="cuda")
    short = torch.empty(100, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), sb.cuda(), pos, cs, n_heads=2, cos_sin_lanes=short)
    with pytest.raises(ValueError):
        gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), sb.cuda(), pos, cs, n_heads=2,
                                        cos_sin_lanes=gpu_lib.rope_table_lanes(cs), scale_rule="ocp_floor")


@pytest.mark.parametrize("M", [8, 1200])
def test_prep_with_lane_copy_bytes_equal(gpu_lib, M):
    """indexer_q_prep with the copy: the one-launch call (8 tokens, which reads
    the table) and the two-call path (1200 tokens, which reads the copy) give
    the bytes of the same call without it."""
    codes, sb = S.weights()
    g = S.rng("indexer_q_m128", 3400 + M)
    x = S.activations_outlier(g, M, 1536).cuda()
    pos = _positions("offset", M, 4096, M).cuda()
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, 4096, 64)
    lanes = gpu_lib.rope_table_lanes(cs)
    q0, s0 = gpu_lib.indexer_q_prep(x, codes.cuda(), sb.cuda(), pos, cs)
    q1, s1 = gpu_lib.indexer_q_prep(x, codes.cuda(), sb.cuda(), pos, cs, cos_sin_lanes=lanes)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1) and torch.equal(s0, s1)
