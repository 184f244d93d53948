"""GPU parity with a RoPE table of other frequencies: every entry point reads
cos / sin from the caller's table, so a rescaled schedule (here a YaRN-style
one: long wavelengths stretched by a factor 4 with a linear ramp between, and
an attention factor folded into cos and sin) needs no kernel change. The
table is built here in float64 and rounded to float32; the oracle takes the
same frequencies and factor in float64. Covered: the pipelined and
small-batch fused kernels, the general kernel (K = 1024), the one-launch
path, the standalone epilogue, and the interleaved variant."""
import math

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C
from oracle import indexer_q as IQ

from gpu_util import oracle_chain_from_x

pytestmark = pytest.mark.gpu

MAX_POS = 4096


def yarn_like_schedule(theta=10000.0, rope_dim=64, factor=4.0, original_ctx=1024, beta_fast=32.0, beta_slow=1.0):
    """Per-pair inverse frequencies and attention factor of a YaRN-style
    context extension (an input recipe: the pages use the plain schedule)."""
    half = rope_dim // 2
    base = theta ** (-2.0 * np.arange(half) / rope_dim)
    rotations = original_ctx * base / (2 * math.pi)        # turns over the original context
    # ramp 1 (keep) for fast pairs (>= beta_fast turns), 0 (stretch) for slow ones (<= beta_slow)
    ramp = np.clip((rotations - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    inv_freq = base * ramp + (base / factor) * (1.0 - ramp)
    mscale = 0.1 * math.log(factor) + 1.0
    return inv_freq, mscale


@pytest.fixture(scope="module")
def schedule():
    inv_freq, mscale = yarn_like_schedule()
    ang = np.arange(MAX_POS, dtype=np.float64)[:, None] * inv_freq[None, :]
    table = np.concatenate([mscale * np.cos(ang), mscale * np.sin(ang)], axis=1).astype(np.float32)
    return {"inv_freq": inv_freq, "mscale": mscale, "table": torch.from_numpy(table).cuda()}


def test_schedule_is_not_the_default(schedule):
    inv_freq, _ = yarn_like_schedule()
    base = 10000.0 ** (-2.0 * np.arange(32) / 64)
    assert inv_freq[0] == base[0] and inv_freq[-1] == base[-1] / 4.0
    assert np.count_nonzero(inv_freq != base) >= 10


@pytest.mark.parametrize("M", [5, 300])
def test_fused_chain_rescaled_table(gpu_lib, schedule, M):
    """M = 5: the small-batch kernel; M = 300: the pipelined kernel."""
    codes, sb = S.weights()
    inp = S.indexer_q_inputs("indexer_q_m128", M=M)
    x, pos = inp["x"], inp["positions"]
    print(f"[rope table] fused M={M}", flush=True)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    q, s = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), sb.cuda(), pos.cuda(), schedule["table"])
    torch.cuda.synchronize()
    ref = oracle_chain_from_x(x, codes, sb, pos, 64, inv_freq=schedule["inv_freq"], mscale=schedule["mscale"])
    rep = C.check_fp4(q.cpu().numpy(), s.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep
    # and the default schedule's oracle does not accept it: the table was used
    plain = oracle_chain_from_x(x, codes, sb, pos, 64)
    assert not C.check_fp4(q.cpu().numpy(), s.cpu().numpy(), plain["z"], plain["q_fp4"], plain["q_scales"])["ok"]


def test_general_kernel_and_interleaved_rescaled_table(gpu_lib, schedule):
    H, M, K = 3, 70, 1024
    codes, sb = S.weights(N=H * 128, K=K, seed=101)
    g = S.rng("indexer_q_m128", 900 + K)
    x = S.activations_outlier(g, M, K)
    pos = S.positions_uniform(g, M, MAX_POS)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    for layout in ("half_split", "interleaved"):
        print(f"[rope table] general K={K} {layout}", flush=True)
        q, s = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, codes.cuda(), sb.cuda(), pos.cuda(), schedule["table"],
                                               n_heads=H, rope_layout=layout)
        torch.cuda.synchronize()
        ref = oracle_chain_from_x(x, codes, sb, pos, H, rope_layout=layout, inv_freq=schedule["inv_freq"],
                                  mscale=schedule["mscale"])
        rep = C.check_fp4(q.cpu().numpy(), s.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
        assert rep["ok"], (layout, rep)


def test_one_launch_rescaled_table(gpu_lib, schedule):
    codes, sb = S.weights()
    inp = S.indexer_q_inputs("indexer_q_m128", M=8)
    x, pos = inp["x"], inp["positions"]
    print("[rope table] one launch M=8", flush=True)
    q, s = gpu_lib.indexer_q_prep_bf16(x.cuda(), codes.cuda(), sb.cuda(), pos.cuda(), schedule["table"])
    torch.cuda.synchronize()
    ref = oracle_chain_from_x(x, codes, sb, pos, 64, inv_freq=schedule["inv_freq"], mscale=schedule["mscale"])
    rep = C.check_fp4(q.cpu().numpy(), s.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep


@pytest.mark.parametrize("layout", ["half_split", "interleaved"])
def test_standalone_epilogue_rescaled_table(gpu_lib, schedule, layout):
    M, H = 37, 3
    inp = S.q_bf16_inputs("indexer_q_m128", M=M, n_heads=H)
    q, pos = inp["q"], inp["positions"]
    print(f"[rope table] epilogue {layout}", flush=True)
    codes, scales = gpu_lib.indexer_q_rope_hadamard_fp4(q.cuda(), pos.cuda(), schedule["table"], n_heads=H,
                                                        rope_layout=layout)
    torch.cuda.synchronize()
    ref = IQ.indexer_q_epilogue(q.float().numpy().astype(np.float64), pos.numpy(), n_heads=H, rope_layout=layout,
                                inv_freq=schedule["inv_freq"], mscale=schedule["mscale"])
    rep = C.check_fp4(codes.cpu().numpy(), scales.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep
