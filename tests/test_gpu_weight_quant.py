"""GPU parity: weight preparation (bf16 [N, K] -> E4M3 codes + one UE8M0 byte
per 128x128 tile), bit-exact against the oracle: a [1024, 1536] matrix in
full, edge tiles (zero, 448 * 2^k, one bf16 step above, the largest bf16,
subnormals, x1e-6), sampled tile rows of the [8192, 1536] projection weight,
strided operands with guard bytes, and the fused kernel fed with the weights
it produces."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C
from oracle import quant_fp8 as QO

from gpu_util import oracle_chain_from_x

pytestmark = pytest.mark.gpu


def bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def check(iqp, w_bf16):
    print(f"[weight quant] {tuple(w_bf16.shape)}", flush=True)
    q, s = iqp.fp8_quant_weight_128x128_ue8m0(w_bf16.cuda())
    torch.cuda.synchronize()
    q_ref, s_ref = QO.fp8_quant_weight_128x128_ue8m0(w_bf16.float().numpy())
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    return q, s


def test_weight_quant_normal_weights(gpu_lib):
    g = np.random.default_rng([100, 7])
    check(gpu_lib, bf16(g.standard_normal((1024, 1536)) * 0.02))


def test_weight_quant_edge_tiles(gpu_lib):
    g = np.random.default_rng([100, 8])
    w = g.uniform(-1, 1, (384, 512)).astype(np.float32)
    w[0:128, 0:128] = 0                                   # floor: byte 105
    w[0:128, 128:256] *= 100.0
    w[5, 140] = 448.0 * 4                                 # amax exactly 448 * 2^2
    w[0:128, 256:384] *= 100.0
    w[9, 300] = -1.75 * 2.0 ** 10 * (1 + 2 ** -7)         # one bf16 step above 448 * 2^2
    w[128:256, 0:128] = np.float32(np.uint32(0x7F7F0000).view(np.float32)) * np.sign(w[128:256, 0:128])
    w[128:256, 128:256] = (np.arange(128 * 128) % 127 + 1).astype(np.uint32).reshape(128, 128)
    w[128:256, 128:256] = (w[128:256, 128:256].astype(np.uint32) << 16).view(np.float32)   # bf16 subnormals
    w[256:384, 0:128] *= 1e-6
    check(gpu_lib, bf16(w))


@pytest.mark.parametrize("N,K", [(128, 128), (256, 128), (640, 896), (1152, 1408)])
def test_weight_quant_tile_counts(gpu_lib, N, K):
    """Tile counts of 1, 2, 35 and 99: workgroups that walk one, two or three
    tiles, and a last workgroup with fewer than the others."""
    g = np.random.default_rng([100, 10, N, K])
    w = g.standard_normal((N, K)) * 0.02 * np.exp2(g.integers(-3, 4, size=(N // 128, 1, K // 128, 1)).repeat(
        128, axis=1).repeat(128, axis=3).reshape(N, K))
    check(gpu_lib, bf16(w))


def test_weight_quant_projection_weight_sampled_tile_rows(gpu_lib):
    g = np.random.default_rng([100, 9])
    w = bf16(g.standard_normal((8192, 1536)) * 0.02)
    q, s = gpu_lib.fp8_quant_weight_128x128_ue8m0(w.cuda())
    torch.cuda.synchronize()
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    for tr in (0, 17, 40, 63):
        rows = slice(128 * tr, 128 * tr + 128)
        q_ref, s_ref = QO.fp8_quant_weight_128x128_ue8m0(w[rows].float().numpy())
        assert np.array_equal(sh[tr], s_ref[0]) and np.array_equal(qh[rows], q_ref), tr


def test_weight_quant_strides_and_guard_bytes(gpu_lib):
    g = np.random.default_rng([100, 10])
    N, K = 256, 384
    w = bf16(g.standard_normal((N, K)))
    wide = torch.zeros((N, K + 64), dtype=torch.bfloat16)
    wide[:, 8:8 + K] = w
    wv = wide.cuda()[:, 8:8 + K]
    qbuf = torch.full((N * (K + 16) + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    qv = qbuf[32:32 + N * (K + 16)].view(N, K + 16)[:, :K]
    sbuf = torch.full((2 * 8 + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    sv = sbuf[32:32 + 16].view(2, 8)[:, :3]
    gpu_lib.fp8_quant_weight_128x128_ue8m0(wv, q=qv, scales=sv)
    qh, sh = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(qh[:32] == 0x5A) and np.all(qh[32 + N * (K + 16):] == 0x5A)
    assert np.all(qh[32:32 + N * (K + 16)].reshape(N, K + 16)[:, K:] == 0x5A)
    assert np.all(sh[:32] == 0xA5) and np.all(sh[48:] == 0xA5)
    assert np.all(sh[32:48].reshape(2, 8)[:, 3:] == 0xA5)
    q_ref, s_ref = QO.fp8_quant_weight_128x128_ue8m0(w.float().numpy())
    assert np.array_equal(qv.cpu().numpy(), q_ref) and np.array_equal(sv.cpu().numpy(), s_ref)


def test_weights_from_the_device_feed_the_fused_kernel(gpu_lib):
    g = np.random.default_rng([100, 11])
    w = bf16(g.standard_normal((8192, 1536)) * 0.02)
    wq, ws = gpu_lib.fp8_quant_weight_128x128_ue8m0(w.cuda())
    inp = S.indexer_q_inputs("indexer_q_m128", M=48)
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, inp["max_pos"], 64)
    q, s = gpu_lib.indexer_q_prep(inp["x"].cuda(), wq, ws, inp["positions"].cuda(), cs)
    torch.cuda.synchronize()
    codes, sb = QO.fp8_quant_weight_128x128_ue8m0(w.float().numpy())
    ref = oracle_chain_from_x(inp["x"], torch.from_numpy(codes), torch.from_numpy(sb), inp["positions"], 64)
    rep = C.check_fp4(q.cpu().numpy(), s.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep
