"""Oracle for packed-UE8M0 FP8 1x128 activation quantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
quantization": Summary (an online FP8 quantizer for DeepGEMM activations whose
UE8M0 scale exponents are packed into int32 words) and Risk and fallback (input
is a contiguous BF16 matrix with K divisible by 128; a tiny-scale floor is kept).

Per row m and 128-element block j:

1. amax = max |x| over the block (exact, order-free);
2. amax is floored at ``AMAX_FLOOR`` (the pages' "tiny-scale floor"; reading:
   an amax floor of 1e-4, equivalently a scale exponent of at least -22);
3. e = ceil(log2(amax / 448)), evaluated exactly, so the scale 2^e is the
   smallest power of two that maps the block into E4M3's range;
4. q = E4M3 RNE of x * 2^-e (exact product; never beyond 448 by step 3);
5. the UE8M0 byte is e + 127; four consecutive block bytes form one int32
   word, block 4w+t in byte t (little-endian); bytes past the last block of a
   row are zero.
"""
import numpy as np

from .formats import E4M3_MAX, ceil_log2_ratio, e4m3_encode_rne, is_bf16_exact

BLOCK = 128
AMAX_FLOOR = 1e-4
BLOCKS_PER_WORD = 4


def block_exponents(x: np.ndarray) -> np.ndarray:
    """Scale exponents e[m, j] for a [M, K] array of bf16 values (K % 128 == 0)."""
    M, K = x.shape
    blocks = np.abs(x.astype(np.float64)).reshape(M, K // BLOCK, BLOCK)
    amax = blocks.max(axis=2)
    amax = np.maximum(amax, AMAX_FLOOR)
    return ceil_log2_ratio(amax, E4M3_MAX)


def pack_scale_bytes(b: np.ndarray) -> np.ndarray:
    """[M, nb] scale bytes -> [M, ceil(nb/4)] int32 words (block 4w+t in byte t)."""
    M, nb = b.shape
    nw = -(-nb // BLOCKS_PER_WORD)
    padded = np.zeros((M, nw * BLOCKS_PER_WORD), dtype=np.uint32)
    padded[:, :nb] = b
    words = np.zeros((M, nw), dtype=np.uint32)
    for t in range(BLOCKS_PER_WORD):
        words |= padded[:, t::BLOCKS_PER_WORD] << np.uint32(8 * t)
    return words.view(np.int32)


def unpack_scale_words(words: np.ndarray, nb: int) -> np.ndarray:
    """Inverse of :func:`pack_scale_bytes` for the first nb blocks."""
    w = np.asarray(words).view(np.uint32)
    M, nw = w.shape
    out = np.zeros((M, nw * BLOCKS_PER_WORD), dtype=np.uint8)
    for t in range(BLOCKS_PER_WORD):
        out[:, t::BLOCKS_PER_WORD] = (w >> np.uint32(8 * t)) & 0xFF
    return out[:, :nb]


def fp8_quant_1x128_ue8m0(x) -> tuple:
    """Quantize a [M, K] bf16 matrix (given as float32 holding bf16 values).

    Returns ``(q, scales)``: q uint8 E4M3 codes [M, K] and scales int32
    [M, ceil(K/512)] in the K-major layout (row m, word w).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be divisible by 128")
    if not is_bf16_exact(x):
        raise ValueError("x must hold bfloat16 values")
    e = block_exponents(x)  # [M, K/128]
    inv = np.ldexp(1.0, -np.repeat(e, BLOCK, axis=1))  # 2^-e per element
    q = e4m3_encode_rne(x.astype(np.float64) * inv)
    scale_bytes = (e + 127).astype(np.uint8)
    return q.reshape(M, K), pack_scale_bytes(scale_bytes)


WEIGHT_TILE = 128


def fp8_quant_weight_128x128_ue8m0(w) -> tuple:
    """Weight preparation: E4M3 codes with one UE8M0 scale per 128x128 tile.

    The pages only say the Q projection is a block-scaled FP8 GEMM
    (tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
    quantization", Summary; TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q
    projection with CuTe DSL", sequence diagram). Reading: DeepSeek-style
    weights with one scale per 128x128 tile, the scale chosen by the same
    steps as the activations' (amax over the tile, the 1e-4 floor, the
    exact e = ceil(log2(amax / 448)), codes E4M3 RNE of w * 2^-e).

    w: [N, K] bf16 values (as float32), N and K multiples of 128. Returns
    ``(q, scales)``: uint8 codes [N, K] and uint8 scale bytes [N/128, K/128].
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D")
    N, K = w.shape
    if N % WEIGHT_TILE or K % WEIGHT_TILE:
        raise ValueError("N and K must be divisible by 128")
    if not is_bf16_exact(w):
        raise ValueError("w must hold bfloat16 values")
    tiles = np.abs(w.astype(np.float64)).reshape(N // WEIGHT_TILE, WEIGHT_TILE, K // WEIGHT_TILE, WEIGHT_TILE)
    amax = np.maximum(tiles.max(axis=(1, 3)), AMAX_FLOOR)              # [N/128, K/128]
    e = ceil_log2_ratio(amax, E4M3_MAX)
    inv = np.ldexp(1.0, -np.repeat(np.repeat(e, WEIGHT_TILE, axis=0), WEIGHT_TILE, axis=1))
    q = e4m3_encode_rne(w.astype(np.float64) * inv)
    return q.reshape(N, K), (e + 127).astype(np.uint8)

