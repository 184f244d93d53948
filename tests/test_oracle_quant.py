"""Pins for the FP8 1x128 UE8M0 quantizer oracle (packed-UE8M0 FP8 online
quantization, tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed
FP8 quantization", Summary and Risk and fallback)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant_fp8 as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_golden_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "fp8_quant_worked_example.json")))
    K = g["K"]
    x = np.zeros((len(g["rows"]), K), dtype=np.float32)
    for r, row in enumerate(g["rows"]):
        for i, v in row["nonzero"]:
            x[r, i] = v
    assert F.is_bf16_exact(x)
    q, s = Q.fp8_quant_1x128_ue8m0(x)
    for r, row in enumerate(g["rows"]):
        want = np.zeros(K, dtype=np.uint8)
        for i, c in row["codes"]:
            want[i] = c
        assert q[r].tolist() == want.tolist()
        assert Q.unpack_scale_words(s[r:r + 1], K // 128)[0].tolist() == row["scale_bytes"]
        assert "%08X" % (int(s[r, 0]) & 0xFFFFFFFF) == row["word_hex"]


def next_bf16_up(v):
    """The next bf16 value above a positive bf16 value."""
    return np.uint32(np.float32(v).view(np.uint32) + 0x10000).view(np.float32)


@pytest.mark.parametrize("k", list(range(-22, 120, 7)) + [119])
def test_power_of_two_boundaries(k):
    """amax = 448*2^k -> byte 127+k with the max code 0x7E; one bf16 step more
    -> byte 128+k."""
    x = np.zeros((2, 128), dtype=np.float32)
    x[0, 5] = 448.0 * 2.0 ** k
    x[1, 5] = next_bf16_up(448.0 * 2.0 ** k)
    q, s = Q.fp8_quant_1x128_ue8m0(x)
    b = Q.unpack_scale_words(s, 1)[:, 0]
    assert b[0] == 127 + k and q[0, 5] == 0x7E
    assert b[1] == 128 + k


def test_floor_equals_min_exponent():
    """The amax floor 1e-4 is the same as clamping the exponent at -22: every
    amax up to 448*2^-22 gets byte 105, the next bf16 value gets 106."""
    vals = bf16([0.0, 1e-30, 1e-6, 3e-6, 9.9e-5, 1e-4, 448 * 2.0 ** -22])
    x = np.zeros((len(vals), 128), dtype=np.float32)
    x[:, 0] = vals
    _, s = Q.fp8_quant_1x128_ue8m0(x)
    assert Q.unpack_scale_words(s, 1)[:, 0].tolist() == [105] * len(vals)
    x2 = np.zeros((1, 128), dtype=np.float32)
    x2[0, 0] = next_bf16_up(448 * 2.0 ** -22)
    assert Q.unpack_scale_words(Q.fp8_quant_1x128_ue8m0(x2)[1], 1)[0, 0] == 106


def test_bf16_subnormals_and_signed_zero():
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 0] = 1.0
    x[0, 1] = np.uint32(0x00010000).view(np.float32)   # smallest positive bf16 subnormal
    x[0, 2] = np.uint32(0x80010000).view(np.float32)   # its negative
    x[0, 3] = -0.0
    q, _ = Q.fp8_quant_1x128_ue8m0(x)
    # amax 1 -> e = -8; 1 * 2^8 = 256 = 1.0 * 2^8 -> 0x78; subnormals -> +-0
    assert q[0, :4].tolist() == [0x78, 0x00, 0x80, 0x80]


def _brute_quant_row(row):
    """Independent pure-Python rendering of the method on one row using exact
    rationals: floor, smallest power of two, nearest-even search."""
    codes, scale_bytes = [], []
    for j in range(len(row) // 128):
        blk = row[128 * j:128 * j + 128]
        amax = max(max(abs(Fraction(float(v))) for v in blk), Fraction(1e-4))
        e = 0
        while amax > 448 * Fraction(2) ** e:
            e += 1
        while amax <= 448 * Fraction(2) ** (e - 1):
            e -= 1
        scale_bytes.append(e + 127)
        for v in blk:
            a = abs(Fraction(float(v))) / Fraction(2) ** e
            best = min(range(127), key=lambda c: (abs(a - Fraction(F.E4M3_POS[c])), c % 2))
            codes.append(best | (0x80 if np.signbit(v) else 0))
    return codes, scale_bytes


def test_matches_exact_rational_bruteforce():
    g = np.random.default_rng(7)
    x = g.standard_normal((3, 256)).astype(np.float32)
    x[0, :128] *= 1e3
    x[1, 128:] *= 1e-6
    x[2, 17] = 0.0
    x = bf16(x)
    q, s = Q.fp8_quant_1x128_ue8m0(x)
    for r in range(3):
        codes, sb = _brute_quant_row(x[r])
        assert Q.unpack_scale_words(s[r:r + 1], 2)[0].tolist() == sb
        assert q[r].tolist() == codes


def test_exhaustive_conversion_domain_vs_torch():
    """Every bf16 pattern times every exponent e in [-22, 120] whose result stays
    within 448: the oracle's code equals torch's float8_e4m3fn cast."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v)].astype(np.float64)
    for e in range(-22, 121):
        t = v * 2.0 ** -e
        t = t[np.abs(t) <= 448]
        got = F.e4m3_encode_rne(t)
        want = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        # float32 holds t exactly unless it underflows; both then give +-0
        assert np.array_equal(got, want), e


def test_invariants_random_blocks():
    g = np.random.default_rng(3)
    x = g.standard_normal((64, 1024)).astype(np.float32)
    x *= np.exp(g.uniform(-20, 20, (64, 8))).repeat(128, axis=1).astype(np.float32)
    x = bf16(x)
    q, s = Q.fp8_quant_1x128_ue8m0(x)
    b = Q.unpack_scale_words(s, 8).astype(np.int64)
    assert b.min() >= 105 and b.max() <= 247
    deq = F.e4m3_decode(q) * np.ldexp(1.0, np.repeat(b - 127, 128, axis=1))
    # error at most half an E4M3 step at that magnitude (step 2^(E-3), subnormal step 2^-9)
    t = np.abs(x.astype(np.float64)) * np.ldexp(1.0, -np.repeat(b - 127, 128, axis=1))
    exp = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
    step = np.ldexp(1.0, (exp - 3).astype(np.int64))
    err = np.abs(deq - x) * np.ldexp(1.0, -np.repeat(b - 127, 128, axis=1))
    assert np.all(err <= step / 2)
    # every block reaches the top binade: its amax maps into (224, 448]
    amax_scaled = t.reshape(64, 8, 128).max(axis=2)
    assert np.all((amax_scaled > 224) | (b == 105))


def test_pack_unpack_roundtrip_and_padding():
    b = np.random.default_rng(0).integers(105, 248, size=(5, 7)).astype(np.uint8)
    w = Q.pack_scale_bytes(b)
    assert w.shape == (5, 2) and w.dtype == np.int32
    assert np.array_equal(Q.unpack_scale_words(w, 7), b)
    assert np.all((w[:, 1].view(np.uint32) >> 24) == 0)   # padding byte of block 7


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        Q.fp8_quant_1x128_ue8m0(np.zeros((2, 100), np.float32))
    with pytest.raises(ValueError):
        Q.fp8_quant_1x128_ue8m0(np.full((1, 128), 1.0 + 2 ** -10, np.float32))


# ----------------------------------------------------------------------------
# Weight preparation: one UE8M0 scale per 128x128 tile
# ----------------------------------------------------------------------------


def S_bf16(x):
    """float values rounded to bf16 (torch's RNE cast), returned as float32."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_weight_quant_worked_example():
    # Tile (0, 0): amax 3.0; 3/448 = 0.0067 lies in (2^-8, 2^-7], e = -7, byte
    # 120. 3 * 2^7 = 384 = 1.5 * 2^8 -> 0x7C; 1.0 * 2^7 = 128 -> 0x70;
    # bf16(0.1) = 0.10009765625, * 2^7 = 12.8125, between 12 (0x54) and 13
    # (0x55), nearer 13 -> 0x55; -2^-7 * 2^7 = -1 -> 0xB8.
    # Tile (0, 1): all zero -> amax floored to 1e-4, e = -22, byte 105.
    # Tile (1, 0): amax 448 -> e = 0, byte 127; 448 -> 0x7E.
    # Tile (1, 1): amax 450 (one bf16 step above 448) -> e = 1, byte 128;
    # 450 / 2 = 225 between 224 (0x76) and 240 (0x77) -> 0x76.
    w = np.zeros((256, 256), dtype=np.float32)
    w[3, 7], w[100, 127], w[0, 0], w[127, 64] = 3.0, 1.0, np.float32(0.10009765625), -2.0 ** -7
    w[128, 5] = 448.0
    w[200, 200] = 450.0
    q, s = Q.fp8_quant_weight_128x128_ue8m0(w)
    assert s.tolist() == [[120, 105], [127, 128]]
    assert (q[3, 7], q[100, 127], q[0, 0], q[127, 64]) == (0x7C, 0x70, 0x55, 0xB8)
    assert q[128, 5] == 0x7E and q[200, 200] == 0x76
    assert np.count_nonzero(q) == 6


def test_weight_quant_tiles_are_independent_and_transpose():
    rng = np.random.default_rng(11)
    w = S_bf16(rng.standard_normal((256, 384)) * 0.02)
    q, s = Q.fp8_quant_weight_128x128_ue8m0(w)
    w2 = w.copy()
    w2[130, 300] = 7.0          # tile (1, 2) only
    q2, s2 = Q.fp8_quant_weight_128x128_ue8m0(w2)
    diff_tiles = {(r // 128, c // 128) for r, c in zip(*np.nonzero(q2 != q))}
    assert diff_tiles == {(1, 2)}
    assert np.array_equal(np.argwhere(s2 != s), [[1, 2]])
    # square tiles: quantizing the transpose gives the transposed result
    qt, st = Q.fp8_quant_weight_128x128_ue8m0(np.ascontiguousarray(w.T))
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def test_weight_quant_reduces_to_row_blocks_when_each_shares_the_tile_max():
    # if every 1x128 block of a tile holds the tile's largest magnitude, the
    # tile exponent equals every block exponent: the 128x128 result is the
    # (independently pinned) 1x128 result
    rng = np.random.default_rng(12)
    w = S_bf16(rng.uniform(-1.0, 1.0, (256, 256)))
    for r in range(256):
        for jb in range(2):
            w[r, 128 * jb + (r * 7 + jb) % 128] = 2.5 if (r // 128 + jb) % 2 else -2.5
    q, s = Q.fp8_quant_weight_128x128_ue8m0(w)
    q1, words = Q.fp8_quant_1x128_ue8m0(w)
    b1 = Q.unpack_scale_words(words, 2)
    assert np.array_equal(q, q1)
    assert np.array_equal(np.repeat(s, 128, axis=0), b1)


def test_weight_quant_rejects_ragged_shapes():
    with pytest.raises(ValueError):
        Q.fp8_quant_weight_128x128_ue8m0(np.zeros((128, 200), dtype=np.float32))
