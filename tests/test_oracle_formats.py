"""Pins for the oracle's number formats (OCP OFP8 E4M3, OCP MX E2M1 / E8M0).

Each encoder is checked against (a) values fixed by the format definitions,
(b) an independent brute-force nearest search written here, and, for E4M3,
(c) torch's CPU float8_e4m3fn cast (a library routine that rounds to nearest
even; agreeing with it on every in-range bf16 value pins the tie rule).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


# ---------------------------------------------------------------- E4M3 table


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0),
    (0x77, 240.0), (0x80, -0.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_e4m3_decode_known_codes(code, value):
    got = F.e4m3_decode(np.array([code], dtype=np.uint8))[0]
    assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value)


def test_e4m3_nan_codes_and_monotone():
    assert np.isnan(F.E4M3_VALUES[0x7F]) and np.isnan(F.E4M3_VALUES[0xFF])
    assert np.all(np.diff(F.E4M3_POS) > 0)
    assert F.E4M3_POS[-1] == 448.0 and len(F.E4M3_POS) == 127
    # every value is an integer multiple of 2^-9 (the GEMM exactness argument relies on it)
    assert np.all(np.mod(F.E4M3_POS * 512, 1) == 0)


def _brute_e4m3(v: float) -> int:
    """Independent nearest search over all 127 magnitudes, exact rationals."""
    a = abs(Fraction(v))
    best = None
    for c in range(127):
        d = abs(a - Fraction(F.E4M3_POS[c]))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_e4m3_encode_matches_bruteforce_sample():
    v = all_bf16_values()
    v = v[np.abs(v) <= 448]
    sample = np.random.default_rng(0).choice(v, 3000, replace=False)
    sample = np.concatenate([sample, [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.5]])
    got = F.e4m3_encode_rne(sample)
    want = np.array([_brute_e4m3(float(x)) for x in sample], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_encode_matches_torch_on_all_in_range_bf16():
    v = all_bf16_values()
    v = v[np.abs(v) <= 448]
    got = F.e4m3_encode_rne(v)
    want = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_ties_go_to_even_code():
    pos = F.E4M3_POS
    for c in range(126):
        mid = (pos[c] + pos[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert F.e4m3_encode_rne(np.array([mid]))[0] == even
        assert F.e4m3_encode_rne(np.array([-mid]))[0] == even | 0x80
        assert F.e4m3_encode_rne(np.array([np.nextafter(mid, 0)]))[0] == c
        assert F.e4m3_encode_rne(np.array([np.nextafter(mid, 1e9)]))[0] == c + 1


def test_e4m3_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.e4m3_encode_rne(np.array([448.5]))
    with pytest.raises(ValueError):
        F.e4m3_encode_rne(np.array([np.nan]))


# ---------------------------------------------------------------- E2M1


def test_e2m1_values_and_roundtrip():
    assert list(F.E2M1_POS) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for code in range(16):
        v = F.e2m1_decode(np.array([code]))[0]
        assert F.e2m1_encode_rne(np.array([v]))[0] == code


@pytest.mark.parametrize("mid,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)])
def test_e2m1_midpoints_and_neighbours(mid, code):
    lo = int(np.searchsorted(F.E2M1_POS, mid) - 1)
    for sign, sbit in ((1.0, 0), (-1.0, 8)):
        assert F.e2m1_encode_rne(np.array([sign * mid]))[0] == code | sbit
        for dt in (np.float64, np.float32):
            below = float(np.nextafter(dt(mid), dt(0)))
            above = float(np.nextafter(dt(mid), dt(100)))
            assert F.e2m1_encode_rne(np.array([sign * below]))[0] == lo | sbit
            assert F.e2m1_encode_rne(np.array([sign * above]))[0] == (lo + 1) | sbit


def test_e2m1_dense_sweep_vs_bruteforce():
    v = np.linspace(-6, 6, 24001)
    got = F.e2m1_encode_rne(v)
    for x, c in zip(v, got):
        a = abs(Fraction(float(x)))
        best = min(range(8), key=lambda k: (abs(a - Fraction(float(F.E2M1_POS[k]))), k % 2))
        assert c == best | (8 if x < 0 or (x == 0 and math.copysign(1, x) < 0) else 0)


def test_e2m1_pack_nibble_order():
    codes = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    packed = F.e2m1_pack(codes)
    assert packed.tolist() == [[0x21, 0x43]]
    assert np.array_equal(F.e2m1_unpack(packed), codes)


# ---------------------------------------------------------------- scales


def test_ue8m0_decode():
    assert F.ue8m0_decode(np.array([127]))[0] == 1.0
    assert F.ue8m0_decode(np.array([0]))[0] == 2.0 ** -127
    assert F.ue8m0_decode(np.array([254]))[0] == 2.0 ** 127
    assert np.isnan(F.ue8m0_decode(np.array([255]))[0])


def _ceil_log2_exact(a: Fraction, d: Fraction) -> int:
    e = 0
    while a > d * Fraction(2) ** e:
        e += 1
    while a <= d * Fraction(2) ** (e - 1):
        e -= 1
    return e


@pytest.mark.parametrize("denom", [448.0, 6.0])
def test_ceil_log2_ratio_vs_exact_rationals(denom):
    g = np.random.default_rng(1)
    a = np.concatenate([
        np.exp(g.uniform(-30, 30, 400)),
        [denom * 2.0 ** k for k in range(-30, 30)],
        [np.nextafter(denom * 2.0 ** k, np.inf) for k in range(-30, 30)],
        [np.nextafter(denom * 2.0 ** k, 0) for k in range(-30, 30)],
        [1e-4, 3.0e38],
    ])
    got = F.ceil_log2_ratio(a, denom)
    want = [_ceil_log2_exact(Fraction(float(x)), Fraction(denom)) for x in a]
    assert got.tolist() == want
