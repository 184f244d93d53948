"""GPU parity: the standalone epilogue (bf16 Q in; RoPE, Hadamard-128, FP4
out) against the oracle's epilogue on the same seeded Q.

The FP4 output is checked with the acceptance rule of the fused path
(relative L2 <= 2e-2 of the dequantized values; a scale byte or a code may
differ only at a rounding boundary, at most 0.1 %). Cases: the 128-token
workload, ragged vector counts (the grid's tail), a strided Q, the pages'
small token counts, the 4,632-token workload (sampled tokens), table-edge
positions, M = 0 and guard bytes around the outputs."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C
from oracle import indexer_q as IQ

pytestmark = pytest.mark.gpu

THETA = S.ROPE_THETA


@pytest.fixture(scope="module")
def tables(gpu_lib):
    return {mp: gpu_lib.rope_cos_sin_table(THETA, mp, 64) for mp in (4096, 4632)}


def oracle_epilogue(q_bf16: torch.Tensor, positions: torch.Tensor, n_heads: int, rope_layout="half_split",
                    scale_rule="ceil") -> dict:
    return IQ.indexer_q_epilogue(q_bf16.float().numpy().astype(np.float64), positions.numpy(),
                                 n_heads=n_heads, rope_layout=rope_layout, scale_rule=scale_rule)


def run_and_check(iqp, q, pos, cs, n_heads, q_dev=None, rope_layout="half_split", scale_rule="ceil"):
    print(f"[epilogue] M={q.shape[0]} H={n_heads} {rope_layout} {scale_rule}", flush=True)
    qd = q.cuda() if q_dev is None else q_dev
    codes, scales = iqp.indexer_q_rope_hadamard_fp4(qd, pos.cuda(), cs, n_heads=n_heads, rope_layout=rope_layout,
                                                    scale_rule=scale_rule)
    torch.cuda.synchronize()
    ref = oracle_epilogue(q, pos, n_heads, rope_layout, scale_rule)
    rep = C.check_fp4(codes.cpu().numpy(), scales.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"],
                      scale_rule=scale_rule)
    assert rep["ok"], rep
    return rep


def test_epilogue_m128(gpu_lib, tables):
    inp = S.q_bf16_inputs("indexer_q_m128")
    rep = run_and_check(gpu_lib, inp["q"], inp["positions"], tables[4096], 64)
    assert rep["rel_l2"] < 2e-2


@pytest.mark.parametrize("M,H", [(1, 1), (1, 64), (4, 64), (5, 64), (8, 64), (37, 3), (63, 1), (129, 5)])
def test_epilogue_ragged(gpu_lib, tables, M, H):
    inp = S.q_bf16_inputs("indexer_q_m128", M=M, n_heads=H)
    run_and_check(gpu_lib, inp["q"], inp["positions"], tables[4096], H)


def test_epilogue_strided_rows(gpu_lib, tables):
    M, H = 40, 3
    inp = S.q_bf16_inputs("indexer_q_m128", M=M, n_heads=H)
    wide = torch.zeros((M, H * 128 + 72), dtype=torch.bfloat16)
    wide[:, 8:8 + H * 128] = inp["q"]
    view = wide.cuda()[:, 8:8 + H * 128]
    assert view.stride(0) == H * 128 + 72
    run_and_check(gpu_lib, inp["q"], inp["positions"], tables[4096], H, q_dev=view)


def test_epilogue_m4632_sampled(gpu_lib, tables):
    inp = S.q_bf16_inputs("indexer_q_m4632")
    q, pos = inp["q"], inp["positions"]
    codes, scales = gpu_lib.indexer_q_rope_hadamard_fp4(q.cuda(), pos.cuda(), tables[4632], n_heads=64)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(16), np.random.default_rng(4632).integers(0, 4632, 480),
                                     np.arange(4632 - 16, 4632)]))
    ref = oracle_epilogue(q[rows], pos[rows], 64)
    rep = C.check_fp4(codes.cpu().numpy()[rows], scales.cpu().numpy()[rows], ref["z"], ref["q_fp4"],
                      ref["q_scales"])
    assert rep["ok"], rep


def test_epilogue_table_edge_positions(gpu_lib, tables):
    M, H = 6, 2
    inp = S.q_bf16_inputs("indexer_q_m128", M=M, n_heads=H)
    pos = torch.tensor([0, 1, 4095, 4094, 2048, 0], dtype=torch.int64)
    run_and_check(gpu_lib, inp["q"], pos, tables[4096], H)


def test_epilogue_empty(gpu_lib, tables):
    q = torch.empty((0, 128 * 64), dtype=torch.bfloat16, device="cuda")
    pos = torch.empty((0,), dtype=torch.int64, device="cuda")
    codes, scales = gpu_lib.indexer_q_rope_hadamard_fp4(q, pos, tables[4096], n_heads=64)
    assert codes.shape == (0, 64, 64) and scales.shape == (0, 64, 4)


def test_epilogue_no_write_outside_outputs(gpu_lib, tables):
    M, H = 7, 3
    inp = S.q_bf16_inputs("indexer_q_m128", M=M, n_heads=H)
    n_codes, n_sc = M * H * 64, M * H * 4
    cbuf = torch.full((n_codes + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((n_sc + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    codes = cbuf[32:32 + n_codes].view(M, H, 64)
    scales = sbuf[32:32 + n_sc].view(M, H, 4)
    gpu_lib.indexer_q_rope_hadamard_fp4(inp["q"].cuda(), inp["positions"].cuda(), tables[4096], n_heads=H,
                                        q_fp4=codes, q_scales=scales)
    ch, sh = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(ch[:32] == 0x5A) and np.all(ch[32 + n_codes:] == 0x5A)
    assert np.all(sh[:32] == 0xA5) and np.all(sh[32 + n_sc:] == 0xA5)
    ref = oracle_epilogue(inp["q"], inp["positions"], H)
    rep = C.check_fp4(codes.cpu().numpy(), scales.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep


VARIANTS = [("interleaved", "ceil"), ("half_split", "ocp_floor"), ("interleaved", "ocp_floor")]


@pytest.mark.parametrize("layout,rule", VARIANTS)
def test_epilogue_variants_m128(gpu_lib, tables, layout, rule):
    inp = S.q_bf16_inputs("indexer_q_m128")
    rep = run_and_check(gpu_lib, inp["q"], inp["positions"], tables[4096], 64, rope_layout=layout,
                        scale_rule=rule)
    assert rep["rel_l2"] < 2e-2


@pytest.mark.parametrize("layout,rule", VARIANTS)
@pytest.mark.parametrize("M,H", [(1, 1), (37, 3), (129, 65)])
def test_epilogue_variants_ragged(gpu_lib, tables, layout, rule, M, H):
    inp = S.q_bf16_inputs("indexer_q_m128", M=M, n_heads=H)
    run_and_check(gpu_lib, inp["q"], inp["positions"], tables[4096], H, rope_layout=layout, scale_rule=rule)


def test_epilogue_variants_differ_from_default(gpu_lib, tables):
    """Each flag changes the output (a variant that ignored its flag would
    pass its parity test only if the two conventions agreed on this input)."""
    inp = S.q_bf16_inputs("indexer_q_m128", M=16, n_heads=4)
    qd, pd = inp["q"].cuda(), inp["positions"].cuda()
    outs = {}
    for layout in ("half_split", "interleaved"):
        for rule in ("ceil", "ocp_floor"):
            c, s = gpu_lib.indexer_q_rope_hadamard_fp4(qd, pd, tables[4096], n_heads=4, rope_layout=layout,
                                                       scale_rule=rule)
            outs[layout, rule] = (c.cpu().numpy(), s.cpu().numpy())
    base_c, base_s = outs["half_split", "ceil"]
    assert not np.array_equal(outs["interleaved", "ceil"][0], base_c)
    assert not np.array_equal(outs["half_split", "ocp_floor"][1], base_s)
    # the floor rule's exponent is never above the ceil rule's: floor(log2 a) - 2 <= ceil(log2(a / 6))
    assert np.all(outs["half_split", "ocp_floor"][1] <= base_s)


def test_epilogue_variant_flags_rejected(gpu_lib, tables):
    inp = S.q_bf16_inputs("indexer_q_m128", M=2, n_heads=1)
    with pytest.raises(ValueError):
        gpu_lib.indexer_q_rope_hadamard_fp4(inp["q"].cuda(), inp["positions"].cuda(), tables[4096], n_heads=1,
                                            rope_layout="neox")


@pytest.mark.parametrize("rule", ["ceil", "ocp_floor"])
def test_epilogue_tiny_and_zero_blocks(gpu_lib, tables, rule):
    """Blocks below the 1e-4 amax floor (all-zero heads, heads of ~1e-7) take
    the floor exponent (-15 by the ceil rule, -16 by the floor rule)."""
    M, H = 9, 4
    inp = S.q_bf16_inputs("indexer_q_m128", M=M, n_heads=H)
    q = inp["q"].clone()
    q[:, 0:128] = 0
    q[:, 128:256] = (q[:, 128:256].float() * 1e-7).to(torch.bfloat16)
    rep = run_and_check(gpu_lib, q, inp["positions"], tables[4096], H, scale_rule=rule)
    assert rep["ok"]
    _, scales = gpu_lib.indexer_q_rope_hadamard_fp4(q.cuda(), inp["positions"].cuda(), tables[4096], n_heads=H,
                                                    scale_rule=rule)
    floor_byte = 127 + (-15 if rule == "ceil" else -16)
    assert np.all(scales.cpu().numpy()[:, 0:2] == floor_byte)


def test_epilogue_variant_m4632_sampled(gpu_lib, tables):
    inp = S.q_bf16_inputs("indexer_q_m4632")
    q, pos = inp["q"], inp["positions"]
    codes, scales = gpu_lib.indexer_q_rope_hadamard_fp4(q.cuda(), pos.cuda(), tables[4632], n_heads=64,
                                                        rope_layout="interleaved", scale_rule="ocp_floor")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(8), np.random.default_rng(4633).integers(0, 4632, 240),
                                     np.arange(4632 - 8, 4632)]))
    ref = oracle_epilogue(q[rows], pos[rows], 64, "interleaved", "ocp_floor")
    rep = C.check_fp4(codes.cpu().numpy()[rows], scales.cpu().numpy()[rows], ref["z"], ref["q_fp4"],
                      ref["q_scales"], scale_rule="ocp_floor")
    assert rep["ok"], rep
