"""Low-precision number formats, written from the public OCP definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* E4M3 ("fn" variant of the OCP 8-bit Floating Point Specification, OFP8 v1.0):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
  encodes subnormals m/8 * 2^-6; there is no infinity; S.1111.111 is NaN; the
  largest finite magnitude is 1.75 * 2^8 = 448.
* E2M1 (OCP Microscaling Formats v1.0, FP4): 1 sign bit, 2 exponent bits with
  bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E8M0 / UE8M0 (same MX document): an unsigned byte b meaning 2^(b-127);
  0xFF is NaN.

The pages name these formats (tokenspeed PR "perf(deepseek-v4): accelerate
indexer Q and packed FP8 quantization", Summary: "packed-UE8M0 FP8", "FP4") but
do not define them; the definitions above are the standard ones.

Rounding to these formats is round-to-nearest with ties to the even encoding,
done here by the plainest possible method: find the two neighbouring
representable magnitudes and pick the nearer; on a tie pick the one whose code
is even (the code's least significant bit is the mantissa's least significant
bit, so "even code" is "even mantissa").
"""
import numpy as np

# ----------------------------------------------------------------------------
# E4M3 (fn)
# ----------------------------------------------------------------------------


def _e4m3_decode_scalar(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** -6
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


#: value of every E4M3 code 0..255 (float64; NaN for 0x7F and 0xFF)
E4M3_VALUES = np.array([_e4m3_decode_scalar(c) for c in range(256)], dtype=np.float64)
#: non-negative finite magnitudes, indexed by code 0..126 (strictly increasing)
E4M3_POS = E4M3_VALUES[:127].copy()
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 E4M3 codes to float64."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne(v) -> np.ndarray:
    """Round float64 values with |v| <= 448 to E4M3 codes (RNE, sign kept).

    Values beyond 448 never occur in this method (the block scale guarantees
    |v| <= 448), so they are rejected rather than given a saturation rule.
    A negative value that rounds to zero gives the negative-zero code 0x80.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("e4m3_encode_rne: input outside [-448, 448]")
    lo = np.searchsorted(E4M3_POS, a, side="right") - 1  # largest code with value <= a
    hi = np.minimum(lo + 1, 126)
    d_lo = a - E4M3_POS[lo]
    d_hi = E4M3_POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


# ----------------------------------------------------------------------------
# E2M1 (MX FP4)
# ----------------------------------------------------------------------------

#: non-negative magnitudes indexed by the 3-bit code 0..7
E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
#: value of every 4-bit code 0..15 (bit 3 is the sign)
E2M1_VALUES = np.concatenate([E2M1_POS, -E2M1_POS])


def e2m1_decode(codes) -> np.ndarray:
    """Decode 4-bit E2M1 codes (0..15) to float64; code 8 is -0.0."""
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode_rne(v) -> np.ndarray:
    """Round float64 values with |v| <= 6 to 4-bit E2M1 codes (RNE, sign kept)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(~np.isfinite(a)) or np.any(a > E2M1_MAX):
        raise ValueError("e2m1_encode_rne: input outside [-6, 6]")
    lo = np.searchsorted(E2M1_POS, a, side="right") - 1
    hi = np.minimum(lo + 1, 7)
    d_lo = a - E2M1_POS[lo]
    d_hi = E2M1_POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def e2m1_pack(codes) -> np.ndarray:
    """Pack 4-bit codes along the last axis, two per byte: element 2t in the
    low nibble, element 2t+1 in the high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("e2m1_pack: odd last dimension")
    return (codes[..., 0::2] & 0xF) | ((codes[..., 1::2] & 0xF) << 4)


def e2m1_unpack(packed) -> np.ndarray:
    """Inverse of :func:`e2m1_pack`."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# ----------------------------------------------------------------------------
# E8M0 (UE8M0) scale bytes
# ----------------------------------------------------------------------------


def ue8m0_decode(b) -> np.ndarray:
    """Scale byte b -> 2^(b-127) as float64 (b = 255 is NaN)."""
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


def ceil_log2_ratio(amax, denom: float) -> np.ndarray:
    """Smallest integer e with amax <= denom * 2^e, for amax > 0.

    This is ceil(log2(amax / denom)) evaluated exactly: a first estimate from
    frexp is corrected by exact comparisons against denom * 2^e (a power-of-two
    multiple of denom is exact in float64 over the whole range used here).
    """
    amax = np.asarray(amax, dtype=np.float64)
    if np.any(amax <= 0) or np.any(~np.isfinite(amax)):
        raise ValueError("ceil_log2_ratio: amax must be positive and finite")
    _, ex = np.frexp(amax / denom)
    e = ex.astype(np.int64)
    for _ in range(3):  # the estimate is off by at most one either way
        too_small = amax > np.ldexp(denom, e)
        e = np.where(too_small, e + 1, e)
        too_big = amax <= np.ldexp(denom, e - 1)
        e = np.where(too_big, e - 1, e)
    assert np.all(amax <= np.ldexp(denom, e)) and np.all(amax > np.ldexp(denom, e - 1))
    return e


def is_bf16_exact(x) -> bool:
    """True when every float32 in x is exactly a bfloat16 value."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return bool(np.all((u & 0xFFFF) == 0))
