"""GPU parity: the GEMM of the production fused kernels in float32.

The FP4 tests check the small-batch, pipelined and split-role kernels end to
end through the acceptance rule. Here the same kernels' K loops (copies,
operand reads, block scales on the matrix cores) are built with the epilogue
replaced by a float32 store of Q (iqp_debug_indexer_q_f32 stage 3, and the
one-launch kernel's twin), and Q is compared element by element with the
oracle's exact GEMM (TensorRT-LLM PR page, sequence diagram: the GEMM result
feeds the RoPE / FP4 epilogue) under the matrix-core error bound.

Token counts: 1 to 256 (small-batch kernel), 300, 1023, 1024, 1157 and 4632
(the split-role build of the pipelined kernel, from 257 tokens; 4632 checked
on sampled tokens), with an odd head count on each of the large kernels."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C
from oracle import quant_fp8 as QO

from gpu_util import mfma_error_bound, oracle_chain_from_x, weights_for_heads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def table(gpu_lib):
    return gpu_lib.rope_cos_sin_table(S.ROPE_THETA, 4632, 64)


def _check_q(out, ref, codes, sb, rows=None):
    """out: float32 [m, H*128] for the oracle's tokens (rows of the batch)."""
    m = ref["q"].shape[0]
    want = ref["q"].reshape(m, -1)
    a_sb = QO.unpack_scale_words(ref["a_words"], 12)
    bound = mfma_error_bound(ref["a_codes"], a_sb, codes.numpy(), sb.numpy()) + 2.0 ** -20 * np.abs(want)
    got = out if rows is None else out[rows]
    err = C.rel_l2(got, want)
    ratio = float(np.max(np.abs(got - want) / bound))
    print(f"rel_l2 {err:.3e}, max |err|/bound {ratio:.3f}")
    assert err <= 2e-4, err
    assert np.all(np.abs(got - want) <= bound), ratio


def _inputs(M, seed, max_pos=4632):
    g = S.rng("indexer_q_m128", 2000 + seed)
    x = S.activations_outlier(g, M, 1536)
    pos = S.positions_uniform(g, M, max_pos)
    return x, pos


@pytest.mark.parametrize("M,H", [(1, 64), (5, 64), (16, 64), (33, 64), (100, 64), (256, 64), (70, 3),
                                 (300, 64), (1023, 64), (300, 3), (1024, 64), (1157, 64), (1157, 3)])
def test_production_kernel_gemm_float32(gpu_lib, table, M, H):
    codes, sb = weights_for_heads(H)
    x, pos = _inputs(M, M + 7 * H)
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    out = gpu_lib.debug_indexer_q_f32(a, a_s, codes.cuda(), sb.cuda(), pos.cuda(), table, 3,
                                      n_heads=H).cpu().numpy()
    _check_q(out, oracle_chain_from_x(x, codes, sb, pos, H), codes, sb)


def test_production_kernel_gemm_float32_m4632_sampled(gpu_lib, table):
    codes, sb = S.weights()
    inp = S.indexer_q_inputs("indexer_q_m4632")
    x, pos = inp["x"], inp["positions"]
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    out = gpu_lib.debug_indexer_q_f32(a, a_s, codes.cuda(), sb.cuda(), pos.cuda(), table, 3).cpu().numpy()
    M = x.shape[0]
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(M, 256, replace=False),
                                     [0, 127, 128, M - 25, M - 1]]))
    _check_q(out, oracle_chain_from_x(x[rows], codes, sb, pos[rows], 64), codes, sb, rows)


def test_production_kernel_gemm_every_element_written(gpu_lib, table):
    """The diagnostic builds store every element of Q once: a NaN-filled
    output has none left, at a ragged size of each large kernel."""
    codes, sb = S.weights()
    for M in (100, 300, 1157):
        x, pos = _inputs(M, 50 + M)
        a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
        out = torch.full((M + 1, 64 * 128), float("nan"), device="cuda")
        gpu_lib.debug_indexer_q_f32(a, a_s, codes.cuda(), sb.cuda(), pos.cuda(), table, 3, out=out[:M])
        o = out.cpu()
        assert not torch.isnan(o[:M]).any(), M
        assert torch.isnan(o[M]).all(), M   # nothing past the last token


@pytest.mark.parametrize("M", [1, 7, 16, 64, 256])
def test_one_launch_kernel_gemm_float32(gpu_lib, table, M):
    """The one-launch kernel quantizes x itself: its Q must be the oracle's
    GEMM of the oracle's own quantization (which the standalone quantizer
    matches bit for bit)."""
    codes, sb = S.weights()
    x, pos = _inputs(M, 300 + M)
    out = gpu_lib.debug_indexer_q_prep_bf16_f32(x.cuda(), codes.cuda(), sb.cuda(), pos.cuda(), table).cpu().numpy()
    _check_q(out, oracle_chain_from_x(x, codes, sb, pos, 64), codes, sb)
