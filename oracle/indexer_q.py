"""Oracle for the fused indexer-Q preparation: block-scaled FP8 Q projection,
RoPE on each head's rope slice, 128-point Hadamard rotation, FP4 quantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The chain follows TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with
CuTe DSL" (sequence diagram: FP8 input and UE8M0 scales go into a GEMM whose
epilogue applies RoPE and writes packed FP4 Q and scales; Description / Paths
compared: the unfused chain is the Q GEMM, an in-place RoPE kernel and an FP4
quantization kernel with scale copies) and tokenspeed PR "perf(deepseek-v4):
accelerate indexer Q and packed FP8 quantization" (Summary: RoPE, FP4
quantization and a Hadamard transform make up indexer-Q preparation).

The pages name these steps without formulas. The readings taken here:

* weights are E4M3 with one UE8M0 scale per 128x128 tile (the pages only say
  the GEMM is block-scaled FP8);
* RoPE rotates pairs (i, i + rope_dim/2) of the first rope_dim dims of each
  head ("half-split" layout), angle pos * theta^(-2i/rope_dim);
* the Hadamard matrix is the Sylvester one, H[r][c] = (-1)^popcount(r & c),
  normalised by 1/sqrt(128) so that it is orthonormal, and it is applied after
  RoPE to all 128 dims of a head;
* FP4 blocks are 32 consecutive dims with a UE8M0 scale 2^e,
  e = ceil(log2(amax / 6)) with amax floored at 1e-4, codes rounded to nearest
  even; two codes per byte, the even element in the low nibble.
"""
import numpy as np

from .formats import (E2M1_MAX, ceil_log2_ratio, e2m1_encode_rne, e2m1_pack,
                      e4m3_decode)

KBLOCK = 128          # K extent of one activation / weight scale block
WBLOCK_N = 128        # N extent of one weight scale block
FP4_BLOCK = 32        # elements per FP4 scale block
FP4_AMAX_FLOOR = 1e-4
HADAMARD_N = 128


# ----------------------------------------------------------------------------
# Block-scaled FP8 GEMM
# ----------------------------------------------------------------------------


def block_scaled_gemm(a_codes, a_scale_bytes, w_codes, w_scale_bytes) -> np.ndarray:
    """Q[m, n] = sum_j 2^(ea[m,j] + ew[n/128, j]) * sum_{k in block j} A[m,k] W[n,k].

    a_codes [M, K] and w_codes [N, K] are E4M3 codes; a_scale_bytes [M, K/128]
    and w_scale_bytes [N/128, K/128] are UE8M0 bytes (one per 128x128 weight
    tile). With w_scale_bytes [N, K/128] (one per weight row and K block, the
    1x128 weight-scale variant) the exponent is ew[n, j] instead.

    Each E4M3 value is an integer multiple of 2^-9 below 2^9, so every product
    is a multiple of 2^-18 and every partial sum of one 128-block stays below
    2^43 such units: the per-block dot products are exact in float64 whatever
    order the matrix product uses. Only the sum over blocks (ascending j)
    rounds.
    """
    A = e4m3_decode(a_codes)
    W = e4m3_decode(w_codes)
    M, K = A.shape
    N = W.shape[0]
    if K % KBLOCK or N % WBLOCK_N or W.shape[1] != K:
        raise ValueError("block_scaled_gemm: bad shapes")
    nb = K // KBLOCK
    sa = np.ldexp(1.0, np.asarray(a_scale_bytes, dtype=np.int64) - 127)      # [M, nb]
    sw = np.ldexp(1.0, np.asarray(w_scale_bytes, dtype=np.int64) - 127)      # [N/128, nb] or [N, nb]
    if sw.shape == (N // WBLOCK_N, nb):
        sw_n = np.repeat(sw, WBLOCK_N, axis=0)                               # [N, nb]
    elif sw.shape == (N, nb):
        sw_n = sw
    else:
        raise ValueError("block_scaled_gemm: weight scales must be [N/128, K/128] or [N, K/128]")
    Q = np.zeros((M, N), dtype=np.float64)
    for j in range(nb):
        ks = slice(j * KBLOCK, (j + 1) * KBLOCK)
        P = A[:, ks] @ W[:, ks].T
        Q += P * sa[:, j:j + 1] * sw_n[None, :, j]
    return Q


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------


def rope_angles(positions, theta: float, rope_dim: int, inv_freq=None) -> np.ndarray:
    """Angles [M, rope_dim/2]: pos * theta^(-2i/rope_dim), in float64; or
    pos * inv_freq[i] when explicit per-pair frequencies are given (a
    rescaled schedule such as YaRN's: the table the kernels read may hold any
    frequencies)."""
    half = rope_dim // 2
    if inv_freq is None:
        i = np.arange(half, dtype=np.float64)
        inv_freq = np.power(float(theta), -2.0 * i / rope_dim)
    inv_freq = np.asarray(inv_freq, dtype=np.float64)
    if inv_freq.shape != (half,):
        raise ValueError("inv_freq must hold rope_dim/2 frequencies")
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope_cos_sin_table(theta: float, max_pos: int, rope_dim: int) -> np.ndarray:
    """[max_pos, rope_dim] table: cos of the angles in the first half of each
    row, sin in the second half (float64)."""
    ang = rope_angles(np.arange(max_pos), theta, rope_dim)
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def rope_half_split(q, positions, theta: float = 10000.0, rope_dim: int = 64, inv_freq=None,
                    mscale: float = 1.0) -> np.ndarray:
    """Rotate each head's first rope_dim dims; q is [M, H, D] float64.

    For i < rope_dim/2: (x_i, x_{i+half}) -> (x_i c - x_{i+half} s,
    x_{i+half} c + x_i s); dims rope_dim..D-1 are unchanged. c and s are
    mscale * cos / sin of the angle (mscale: an attention factor folded into
    the table, 1 by default), the angle from rope_angles.
    """
    q = np.asarray(q, dtype=np.float64)
    half = rope_dim // 2
    ang = rope_angles(positions, theta, rope_dim, inv_freq)
    c = mscale * np.cos(ang)[:, None, :]
    s = mscale * np.sin(ang)[:, None, :]
    out = q.copy()
    x1 = q[..., :half]
    x2 = q[..., half:rope_dim]
    out[..., :half] = x1 * c - x2 * s
    out[..., half:rope_dim] = x2 * c + x1 * s
    return out


def rope_interleaved(q, positions, theta: float = 10000.0, rope_dim: int = 64, inv_freq=None,
                     mscale: float = 1.0) -> np.ndarray:
    """The interleaved RoPE layout: pair i < rope_dim/2 is dims (2i, 2i + 1),
    rotated by the same angle pos * theta^(-2i/rope_dim); dims rope_dim..D-1
    are unchanged. q is [M, H, D] float64.

    A convention variant: the pages leave the pair layout open (tokenspeed PR
    "perf(deepseek-v4): accelerate indexer Q and packed FP8 quantization",
    Summary, names only an MLA RoPE kernel); both common layouts are offered.
    """
    q = np.asarray(q, dtype=np.float64)
    ang = rope_angles(positions, theta, rope_dim, inv_freq)
    c = mscale * np.cos(ang)[:, None, :]
    s = mscale * np.sin(ang)[:, None, :]
    out = q.copy()
    x1 = q[..., 0:rope_dim:2]
    x2 = q[..., 1:rope_dim:2]
    out[..., 0:rope_dim:2] = x1 * c - x2 * s
    out[..., 1:rope_dim:2] = x2 * c + x1 * s
    return out


# ----------------------------------------------------------------------------
# Hadamard
# ----------------------------------------------------------------------------


def hadamard_matrix(n: int = HADAMARD_N) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix, H[r][c] = (-1)^popcount(r & c)."""
    r = np.arange(n)[:, None]
    c = np.arange(n)[None, :]
    bits = r & c
    pop = np.zeros_like(bits)
    for b in range(int(n).bit_length()):
        pop += (bits >> b) & 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def hadamard_rotate(y) -> np.ndarray:
    """z = (H / sqrt(128)) y along the last axis, as a dense matrix product."""
    y = np.asarray(y, dtype=np.float64)
    H = hadamard_matrix(y.shape[-1])
    return (y @ H.T) / np.sqrt(float(y.shape[-1]))


# ----------------------------------------------------------------------------
# FP4 e2m1 with UE8M0 block scales
# ----------------------------------------------------------------------------


def fp4_quantize(z, decide_dtype=None, scale_rule: str = "ceil") -> tuple:
    """Quantize the last axis (a multiple of 32) in 32-element blocks.

    The scale and code decisions are taken exactly on the float64 z (the
    pages fix no precision for them: they only note that evaluation order can
    move a value across an FP4 rounding boundary, tokenspeed PR
    "perf(deepseek-v4): accelerate indexer Q and packed FP8 quantization",
    Risk and fallback). ``decide_dtype`` (e.g. np.float32) rounds z to that
    type first, for diagnostics. Returns ``(packed, scale_bytes)``: packed
    codes [..., n/2] uint8 and scale bytes [..., n/32] uint8.

    scale_rule "ceil" (the default reading): e = ceil(log2(amax / 6)), the
    smallest power of two that keeps the block within E2M1's range, so codes
    never saturate. "ocp_floor": the OCP MX rule, e = floor(log2 amax) - 2
    (2 being E2M1's largest exponent), codes saturating at +-6. Both floor
    amax at 1e-4 first.
    """
    if scale_rule not in ("ceil", "ocp_floor"):
        raise ValueError(scale_rule)
    z = np.asarray(z, dtype=np.float64)
    if decide_dtype is not None:
        z = z.astype(decide_dtype).astype(np.float64)
    n = z.shape[-1]
    if n % FP4_BLOCK:
        raise ValueError("fp4_quantize: last axis must be a multiple of 32")
    blocks = z.reshape(z.shape[:-1] + (n // FP4_BLOCK, FP4_BLOCK))
    amax = np.maximum(np.abs(blocks).max(axis=-1), FP4_AMAX_FLOOR)
    if scale_rule == "ceil":
        e = ceil_log2_ratio(amax, E2M1_MAX)
    else:
        e = np.frexp(amax)[1].astype(np.int64) - 1 - 2     # frexp: amax = f 2^k, f in [0.5, 1)
    scaled = blocks * np.ldexp(1.0, -e)[..., None]
    scaled = np.clip(scaled, -E2M1_MAX, E2M1_MAX)          # saturation (reached only by "ocp_floor")
    codes = e2m1_encode_rne(scaled).reshape(z.shape)
    return e2m1_pack(codes), (e + 127).astype(np.uint8)


# ----------------------------------------------------------------------------
# Standalone epilogue (the unfused chain's second half)
# ----------------------------------------------------------------------------


def indexer_q_epilogue(q, positions, n_heads: int = 64, head_dim: int = 128, rope_dim: int = 64,
                       theta: float = 10000.0, rope_layout: str = "half_split",
                       scale_rule: str = "ceil", inv_freq=None, mscale: float = 1.0) -> dict:
    """RoPE, Hadamard rotation and FP4 quantization of an already projected Q.

    This is the unfused chain's epilogue (TensorRT-LLM PR "Fuse DeepSeek-V4
    Indexer Q projection with CuTe DSL", Description / Paths compared: the Q
    GEMM writes a bf16 Q that a RoPE kernel and an FP4 quantization kernel then
    consume). q is [M, H*D] (the bf16 values, widened exactly); the steps are
    the same functions the fused chain applies after its GEMM. rope_layout
    ("half_split" or "interleaved") and scale_rule ("ceil" or "ocp_floor")
    select the convention variants; inv_freq / mscale give an explicit
    frequency schedule (rope_angles).
    """
    q = np.asarray(q, dtype=np.float64)
    M = q.shape[0]
    q = q.reshape(M, n_heads, head_dim)
    if rope_layout == "half_split":
        q_rope = rope_half_split(q, positions, theta, rope_dim, inv_freq, mscale)
    elif rope_layout == "interleaved":
        q_rope = rope_interleaved(q, positions, theta, rope_dim, inv_freq, mscale)
    else:
        raise ValueError(rope_layout)
    z = hadamard_rotate(q_rope)
    packed, scales = fp4_quantize(z, scale_rule=scale_rule)
    return {"q_rope": q_rope, "z": z, "q_fp4": packed, "q_scales": scales}


# ----------------------------------------------------------------------------
# Whole chain
# ----------------------------------------------------------------------------


def indexer_q_chain(a_codes, a_scale_bytes, w_codes, w_scale_bytes, positions,
                    n_heads: int = 64, head_dim: int = 128, rope_dim: int = 64,
                    theta: float = 10000.0, rope_layout: str = "half_split",
                    scale_rule: str = "ceil", inv_freq=None, mscale: float = 1.0) -> dict:
    """The whole indexer-Q preparation for one batch of tokens.

    Returns a dict with ``q_fp4`` [M, H, D/2] uint8, ``q_scales`` [M, H, D/32]
    uint8, and the float64 intermediates ``q`` (GEMM output, [M, H, D]),
    ``q_rope`` and ``z`` (the Hadamard-rotated values that were quantized).
    rope_layout ("half_split" or "interleaved") and scale_rule ("ceil" or
    "ocp_floor") select the convention variants, as in indexer_q_epilogue;
    inv_freq / mscale give an explicit frequency schedule (rope_angles).
    """
    M = np.asarray(a_codes).shape[0]
    q = block_scaled_gemm(a_codes, a_scale_bytes, w_codes, w_scale_bytes)
    q = q.reshape(M, n_heads, head_dim)
    if rope_layout == "half_split":
        q_rope = rope_half_split(q, positions, theta, rope_dim, inv_freq, mscale)
    elif rope_layout == "interleaved":
        q_rope = rope_interleaved(q, positions, theta, rope_dim, inv_freq, mscale)
    else:
        raise ValueError(rope_layout)
    z = hadamard_rotate(q_rope)
    packed, scales = fp4_quantize(z, scale_rule=scale_rule)
    return {"q": q, "q_rope": q_rope, "z": z, "q_fp4": packed, "q_scales": scales}
