"""Acceptance rules that compare a device result with the oracle's.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* FP8 quantization: the E4M3 bytes and the packed scale words must be
  identical to the oracle's.
* FP4 indexer-Q: the device holds Q in float32 where the oracle holds it in
  float64, so a value that sits on an FP4 rounding boundary may legitimately
  round the other way (tokenspeed PR "perf(deepseek-v4): accelerate indexer Q
  and packed FP8 quantization", Risk and fallback: evaluation order can give
  rare FP4 rounding-boundary differences). The rule:

  1. relative L2 of the dequantized outputs <= 2e-2;
  2. a scale byte may differ only by one and only where the oracle's block
     amax/6 lies within 2^-10 (relative) of a power of two; at most 0.1 % of
     blocks may differ;
  3. a code may differ only to an adjacent E2M1 value and only where the
     oracle's scaled value lies within 2^-10 of the midpoint between the two
     values (codes are compared at the device's scale for a block whose
     scale legitimately differs); at most 0.1 % of codes may differ.

  The 0.1 % limits are rates: on a sample of fewer than 1000 blocks (or
  codes) they would forbid even one boundary difference, so one legal
  difference is always allowed.
     +0 and -0 are the same value.
"""
import numpy as np

from .formats import E2M1_MAX, E2M1_VALUES, e2m1_unpack
from .indexer_q import FP4_AMAX_FLOOR, FP4_BLOCK

WINDOW = 2.0 ** -10
MAX_FRACTION = 1e-3
REL_L2_TOL = 2e-2

#: the 15 distinct E2M1 values in ascending order (+0 and -0 merged)
_LADDER = np.unique(E2M1_VALUES)


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def check_fp8_quant(q_dev, s_dev, q_ref, s_ref) -> dict:
    """Bit-exact comparison; returns counts of differing bytes and words."""
    q_dev = np.asarray(q_dev).view(np.uint8)
    q_ref = np.asarray(q_ref).view(np.uint8)
    s_dev = np.asarray(s_dev).view(np.int32)
    s_ref = np.asarray(s_ref).view(np.int32)
    if q_dev.shape != q_ref.shape or s_dev.shape != s_ref.shape:
        raise ValueError("check_fp8_quant: shape mismatch")
    nq = int(np.count_nonzero(q_dev != q_ref))
    ns = int(np.count_nonzero(s_dev != s_ref))
    return {"q_mismatch": nq, "scale_mismatch": ns, "ok": nq == 0 and ns == 0}


def _value_index(v):
    return np.searchsorted(_LADDER, v)


def dequant_fp4(packed, scale_bytes) -> np.ndarray:
    """[..., n/2] packed codes + [..., n/32] scale bytes -> float64 [..., n]."""
    codes = e2m1_unpack(packed)
    vals = E2M1_VALUES[codes]
    sb = np.asarray(scale_bytes, dtype=np.int64)
    scale = np.repeat(np.ldexp(1.0, sb - 127), FP4_BLOCK, axis=-1)
    return vals * scale


def check_fp4(q_dev, s_dev, z_ref, q_ref, s_ref, scale_rule: str = "ceil") -> dict:
    """Apply the FP4 acceptance rule.

    q_dev / q_ref: packed codes [..., 64]; s_dev / s_ref: scale bytes [..., 4];
    z_ref: the oracle's float64 values before quantization [..., 128].
    scale_rule: "ceil" (e = ceil(log2(amax / 6)): the exponent steps where
    amax / 6 crosses a power of two) or "ocp_floor" (e = floor(log2 amax) - 2:
    it steps where amax crosses a power of two).
    """
    if scale_rule not in ("ceil", "ocp_floor"):
        raise ValueError(scale_rule)
    q_dev = np.asarray(q_dev, dtype=np.uint8)
    q_ref = np.asarray(q_ref, dtype=np.uint8)
    s_dev = np.asarray(s_dev, dtype=np.uint8).astype(np.int64)
    s_ref = np.asarray(s_ref, dtype=np.uint8).astype(np.int64)
    z = np.asarray(z_ref, dtype=np.float64)
    n = z.shape[-1]
    nblk = n // FP4_BLOCK
    zb = z.reshape(z.shape[:-1] + (nblk, FP4_BLOCK))
    report = {}

    # 1. relative L2 of dequantized values
    dq_dev = dequant_fp4(q_dev, s_dev)
    dq_ref = dequant_fp4(q_ref, s_ref)
    report["rel_l2"] = rel_l2(dq_dev, dq_ref)

    # 2. scale bytes
    amax = np.maximum(np.abs(zb).max(axis=-1), FP4_AMAX_FLOOR)
    ratio = amax / (E2M1_MAX if scale_rule == "ceil" else 4.0)
    nearest_pow2 = np.ldexp(1.0, np.round(np.log2(ratio)).astype(np.int64))
    near_boundary = np.abs(ratio / nearest_pow2 - 1.0) <= WINDOW
    s_diff = s_dev != s_ref
    s_legal = (np.abs(s_dev - s_ref) == 1) & near_boundary
    report["blocks"] = int(s_ref.size)
    report["scale_mismatch"] = int(np.count_nonzero(s_diff))
    report["scale_illegal"] = int(np.count_nonzero(s_diff & ~s_legal))

    # 3. codes, compared at the device's scale
    e_dev = s_dev - 127
    scaled = zb * np.ldexp(1.0, -e_dev)[..., None]
    # clipping a saturating value (floor rule) changes no verdict: beyond +-6
    # the nearest E2M1 value is +-6 either way and no midpoint is near
    scaled = np.clip(scaled, -E2M1_MAX, E2M1_MAX).reshape(z.shape)
    v_dev = E2M1_VALUES[e2m1_unpack(q_dev)]
    # reference value at the device's scale: where the scale agrees this is
    # the oracle's own code; elsewhere requantize the oracle's value
    v_ref_own = E2M1_VALUES[e2m1_unpack(q_ref)]
    same_scale = np.repeat(~s_diff, FP4_BLOCK, axis=-1)
    ladder_idx = np.clip(np.searchsorted(_LADDER, scaled), 0, len(_LADDER) - 1)
    lo = _LADDER[np.clip(ladder_idx - 1, 0, len(_LADDER) - 1)]
    hi = _LADDER[ladder_idx]
    nearest = np.where(np.abs(scaled - lo) <= np.abs(hi - scaled), lo, hi)
    v_ref = np.where(same_scale, v_ref_own, nearest)
    differs = v_dev != v_ref          # -0 == +0 as floats
    i_dev = _value_index(v_dev)
    i_ref = _value_index(v_ref)
    adjacent = np.abs(i_dev - i_ref) == 1
    midpoint = 0.5 * (v_dev + v_ref)
    on_boundary = np.abs(scaled - midpoint) <= WINDOW
    legal = adjacent & on_boundary
    report["codes"] = int(v_dev.size)
    report["code_mismatch"] = int(np.count_nonzero(differs))
    report["code_illegal"] = int(np.count_nonzero(differs & ~legal))

    report["ok"] = bool(
        report["rel_l2"] <= REL_L2_TOL
        and report["scale_illegal"] == 0
        and report["scale_mismatch"] <= max(1.0, MAX_FRACTION * report["blocks"])
        and report["code_illegal"] == 0
        and report["code_mismatch"] <= max(1.0, MAX_FRACTION * report["codes"])
    )
    return report
