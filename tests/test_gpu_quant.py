"""GPU parity: packed-UE8M0 FP8 quantizer, bit-exact against the oracle.

Covers the workload shapes (indexer activations [128, 1536], the standalone
[4632, 7168] matrix with 1 % x1e3 and 1 % x1e-6 blocks, the long-prefill
Student-t matrix sampled by rows), both scale layouts, ragged K (partial
scale words), M = 1, an exhaustive sweep of every bf16 pattern at every scale
exponent, and that every output byte is written."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C
from oracle import quant_fp8 as QO

from gpu_util import bf16_to_np, exhaustive_quant_rows

pytestmark = pytest.mark.gpu


def run_and_compare(iqp, x: torch.Tensor, layout: str = "k"):
    xd = x.cuda()
    q, s = iqp.fp8_quant_1x128_ue8m0(xd, scale_layout=layout)
    torch.cuda.synchronize()
    q_ref, s_ref = QO.fp8_quant_1x128_ue8m0(bf16_to_np(x))
    rep = C.check_fp8_quant(q.cpu().numpy(), s.cpu().contiguous().numpy(), q_ref, s_ref)
    assert rep["ok"], rep
    return q, s


@pytest.mark.parametrize("layout", ["k", "mn"])
def test_indexer_activations_m128(gpu_lib, layout):
    x = S.indexer_q_inputs("indexer_q_m128")["x"]
    run_and_compare(gpu_lib, x, layout)


@pytest.mark.parametrize("layout", ["k", "mn"])
def test_standalone_4632x7168_full(gpu_lib, layout):
    x = S.quant_input("quant_4632x7168")
    run_and_compare(gpu_lib, x, layout)


def test_prefill_32768x7168_sampled_rows(gpu_lib):
    x = S.quant_input("prefill_m32768")
    q, s = gpu_lib.fp8_quant_1x128_ue8m0(x.cuda())
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(x.shape[0], 512, replace=False)
    rows = np.concatenate([rows, [0, x.shape[0] - 1]])
    q_ref, s_ref = QO.fp8_quant_1x128_ue8m0(bf16_to_np(x[rows]))
    rep = C.check_fp8_quant(q.cpu().numpy()[rows], s.cpu().numpy()[rows], q_ref, s_ref)
    assert rep["ok"], rep


@pytest.mark.parametrize("M,K", [(1, 128), (1, 1536), (7, 640), (33, 384), (5, 896), (130, 7168), (3, 2176)])
def test_ragged_shapes(gpu_lib, M, K):
    g = np.random.default_rng(M * 100003 + K)
    x = g.standard_normal((M, K)).astype(np.float32)
    x *= np.exp(g.uniform(-12, 12, (M, K // 128))).repeat(128, axis=1).astype(np.float32)
    run_and_compare(gpu_lib, S.to_bf16(x), "k")
    run_and_compare(gpu_lib, S.to_bf16(x), "mn")


def test_exhaustive_bf16_patterns_every_exponent(gpu_lib):
    rows = exhaustive_quant_rows()
    pad = (-len(rows)) % 8
    rows = np.concatenate([rows, np.zeros((pad, 128), np.float32)])
    x = S.to_bf16(rows.reshape(-1, 1024))
    run_and_compare(gpu_lib, x, "k")


def test_edge_blocks(gpu_lib):
    x = np.zeros((4, 512), dtype=np.float32)
    x[0, 0] = 3.0                                                 # ordinary block
    x[0, 256] = 448.0                                              # exact power-of-two boundary
    x[0, 384] = np.uint32(0x43E10000).view(np.float32)             # one bf16 step above 448
    x[1, :128] = np.uint32(0x00010000).view(np.float32)            # subnormal block
    x[1, 128] = -0.0
    x[2, :] = np.uint32(0x7F7F0000).view(np.float32)               # largest bf16 everywhere
    x[3, 5] = -1e-6
    x[3, 130] = 1.0
    x[3, 131] = -1.0
    run_and_compare(gpu_lib, S.to_bf16(x), "k")


def test_every_output_byte_written(gpu_lib):
    x = S.indexer_q_inputs("indexer_q_m128")["x"].cuda()
    outs = []
    for fill in (0x00, 0xFF):
        q = torch.full((x.shape[0], x.shape[1]), fill, dtype=torch.uint8, device="cuda")
        s = torch.full((x.shape[0], 3), -1 if fill else 0, dtype=torch.int32, device="cuda")
        gpu_lib.fp8_quant_1x128_ue8m0(x, q=q, scales=s)
        outs.append((q.cpu(), s.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_no_write_outside_outputs(gpu_lib):
    """Canary bytes around q and the scale words stay untouched (ragged row
    stride and a partial scale word)."""
    M, K, ldq = 9, 640, 648
    x = S.to_bf16(np.random.default_rng(1).standard_normal((M, K)).astype(np.float32)).cuda()
    qbuf = torch.full((M * ldq + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    q = qbuf[32:32 + M * ldq].view(M, ldq)[:, :K]
    sbuf = torch.full((M * 3 + 8,), 0x13572468, dtype=torch.int32, device="cuda")
    s = sbuf[4:4 + M * 3].view(M, 3)[:, :2]
    gpu_lib.fp8_quant_1x128_ue8m0(x, q=q, scales=s)
    qh = qbuf.cpu().numpy()
    assert np.all(qh[:32] == 0x5A) and np.all(qh[32 + M * ldq:] == 0x5A)
    body = qh[32:32 + M * ldq].reshape(M, ldq)
    assert np.all(body[:, K:] == 0x5A)
    sh = sbuf.cpu().numpy()
    assert np.all(sh[:4] == 0x13572468) and np.all(sh[4 + M * 3:] == 0x13572468)
    assert np.all(sh[4:4 + M * 3].reshape(M, 3)[:, 2] == 0x13572468)
    q_ref, s_ref = QO.fp8_quant_1x128_ue8m0(bf16_to_np(x.cpu()))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)
