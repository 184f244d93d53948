"""Helpers shared by the GPU parity tests: run the oracle on the same seeded
inputs the device path gets, and build inputs with exact properties."""
import numpy as np
import torch

from oracle import formats as F
from oracle import indexer_q as IQ
from oracle import quant_fp8 as QO

import synthetic as S


def bf16_to_np(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy()


def oracle_chain_from_x(x_bf16: torch.Tensor, w_codes: torch.Tensor, w_sb: torch.Tensor,
                        positions: torch.Tensor, n_heads: int, rope_layout: str = "half_split",
                        scale_rule: str = "ceil", **rope) -> dict:
    """The oracle's whole chain (its own FP8 quantization, then the fused
    stages); rope: inv_freq / mscale of an explicit frequency schedule."""
    xn = bf16_to_np(x_bf16)
    a_codes, a_words = QO.fp8_quant_1x128_ue8m0(xn)
    a_sb = QO.unpack_scale_words(a_words, xn.shape[1] // 128)
    out = IQ.indexer_q_chain(a_codes, a_sb, w_codes.numpy(), w_sb.numpy(), positions.numpy(),
                             n_heads=n_heads, rope_layout=rope_layout, scale_rule=scale_rule, **rope)
    out["a_codes"] = a_codes
    out["a_words"] = a_words
    return out


def weights_for_heads(n_heads: int):
    """The standard synthetic weights, cut to the first n_heads heads."""
    codes, sb = S.weights()
    return codes[: n_heads * 128].contiguous(), sb[:n_heads].contiguous()


def exhaustive_quant_rows() -> np.ndarray:
    """Rows of 128 bf16 values covering every (bf16 pattern, exponent e) pair
    whose scaled value stays within E4M3 range: each row has one anchor element
    whose magnitude fixes the block exponent to e, and 127 payload values with
    |x| <= anchor. Returns float32 [rows, 128] holding bf16 values."""
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    finite = bits[np.isfinite(bits)]
    rows = []
    for e in range(-22, 121):
        if e <= 119:
            anchor = np.float32(448.0 * 2.0 ** e)
        else:
            anchor = np.uint32(0x7F7F0000).view(np.float32)    # largest bf16, exponent 120
        payload = finite[np.abs(finite) <= anchor]
        n = -(-len(payload) // 127)
        padded = np.zeros(n * 127, dtype=np.float32)
        padded[: len(payload)] = payload
        blk = np.empty((n, 128), dtype=np.float32)
        blk[:, 0] = anchor
        blk[:, 1:] = padded.reshape(n, 127)
        rows.append(blk)
    return np.concatenate(rows)


def mfma_error_bound(a_codes, a_sb, w_codes, w_sb):
    """Per-element bound on |Q_device - Q_exact| for the FP8 matrix cores.

    Measured on gfx950: one 64-deep FP8 MFMA returns its dot product with an
    error of at most about 2^-11.3 of the largest product term (median 2^-14.5;
    every FP8 MFMA form behaves alike), i.e. products are summed at a fixed
    precision below the largest one rather than in float32. The bound allows
    2^-9 (64 terms x 2^-15) of max|A| * max|W| per 64-deep chunk, times the
    block scales, plus float32 rounding of the running sum.
    """
    A = F.e4m3_decode(a_codes)
    W = F.e4m3_decode(w_codes)
    M, K = A.shape
    nc = K // 64
    amax = np.abs(A).reshape(M, nc, 64).max(-1) * np.repeat(np.ldexp(1.0, a_sb.astype(np.int64) - 127), 2, axis=1)
    wsc = np.repeat(np.repeat(np.ldexp(1.0, w_sb.astype(np.int64) - 127), 128, axis=0), 2, axis=1)
    wmax = np.abs(W).reshape(W.shape[0], nc, 64).max(-1) * wsc
    return 2.0 ** -9 * (amax @ wmax.T)
