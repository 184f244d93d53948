"""Pins for the indexer-Q oracle: block-scaled FP8 GEMM, RoPE, Hadamard-128 and
FP4 e2m1 quantization (TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection
with CuTe DSL", sequence diagram; tokenspeed PR "perf(deepseek-v4): accelerate
indexer Q and packed FP8 quantization", Summary)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import indexer_q as IQ

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E4M3_FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def rand_codes(g, shape):
    return g.choice(E4M3_FINITE, size=shape)


# ---------------------------------------------------------------- GEMM


def test_gemm_one_hot_weights_give_dequantized_activations():
    g = np.random.default_rng(0)
    M, K, N = 5, 256, 128
    a = rand_codes(g, (M, K))
    sa = g.integers(110, 140, size=(M, K // 128)).astype(np.uint8)
    w = np.zeros((N, K), dtype=np.uint8)
    cols = g.integers(0, K, size=N)
    w[np.arange(N), cols] = 0x38          # 1.0
    sw = np.full((1, K // 128), 127, dtype=np.uint8)
    Qm = IQ.block_scaled_gemm(a, sa, w, sw)
    deq = F.e4m3_decode(a) * np.ldexp(1.0, np.repeat(sa.astype(np.int64) - 127, 128, axis=1))
    assert np.array_equal(Qm, deq[:, cols])


def _exact_gemm(a, sa, w, sw):
    """Pure-Python exact rational GEMM: integer block dots times powers of two."""
    M, K = a.shape
    N = w.shape[0]
    A = [[Fraction(float(v)) for v in F.e4m3_decode(r)] for r in a]
    W = [[Fraction(float(v)) for v in F.e4m3_decode(r)] for r in w]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for j in range(K // 128):
                dot = sum(A[m][k] * W[n][k] for k in range(128 * j, 128 * j + 128))
                tot += dot * Fraction(2) ** (int(sa[m, j]) - 127) * Fraction(2) ** (int(sw[n // 128, j]) - 127)
            out[m][n] = tot
    return out


def test_gemm_vs_exact_rationals():
    g = np.random.default_rng(1)
    M, K, N = 3, 384, 256
    a = rand_codes(g, (M, K))
    w = rand_codes(g, (N, K))
    sa = g.integers(100, 150, size=(M, K // 128)).astype(np.uint8)
    sw = g.integers(100, 150, size=(N // 128, K // 128)).astype(np.uint8)
    got = IQ.block_scaled_gemm(a, sa, w, sw)
    want = _exact_gemm(a, sa, w, sw)
    for m in range(M):
        for n in range(0, N, 7):
            exact = want[m][n]
            # only the 3-term sum over blocks rounds: relative error <= 3 * 2^-53
            assert abs(Fraction(float(got[m, n])) - exact) <= abs(exact) * Fraction(3, 2 ** 53) + Fraction(1, 2 ** 200)


def test_gemm_k128_is_one_scaled_integer_dot():
    g = np.random.default_rng(2)
    a = rand_codes(g, (4, 128))
    w = rand_codes(g, (128, 128))
    sa = np.array([[120], [127], [130], [140]], dtype=np.uint8)
    sw = np.array([[125]], dtype=np.uint8)
    got = IQ.block_scaled_gemm(a, sa, w, sw)
    ai = np.round(F.e4m3_decode(a) * 512).astype(np.int64)     # integers (units of 2^-9)
    wi = np.round(F.e4m3_decode(w) * 512).astype(np.int64)
    dots = ai @ wi.T                                             # exact int64
    want = np.ldexp(dots.astype(np.float64), (sa.astype(np.int64) - 127 + 125 - 127 - 18))
    assert np.array_equal(got, want)


def test_gemm_matches_numpy_float64_on_small_shape():
    g = np.random.default_rng(3)
    a = rand_codes(g, (6, 256))
    w = rand_codes(g, (128, 256))
    sa = np.full((6, 2), 127, np.uint8)
    sw = np.full((1, 2), 127, np.uint8)
    got = IQ.block_scaled_gemm(a, sa, w, sw)
    want = np.matmul(F.e4m3_decode(a), F.e4m3_decode(w).T)
    assert np.allclose(got, want, rtol=1e-15, atol=0)


def test_gemm_weight_scale_applies_per_128_rows():
    g = np.random.default_rng(4)
    a = rand_codes(g, (2, 128))
    w = rand_codes(g, (256, 128))
    sa = np.full((2, 1), 127, np.uint8)
    base = IQ.block_scaled_gemm(a, sa, w, np.array([[127], [127]], np.uint8))
    moved = IQ.block_scaled_gemm(a, sa, w, np.array([[127], [130]], np.uint8))
    assert np.array_equal(moved[:, :128], base[:, :128])
    assert np.array_equal(moved[:, 128:], base[:, 128:] * 8)


def test_gemm_weight_scales_per_row_closed_form():
    # A = [1, 2] in block 0 and [3] in block 1 (E4M3 1.0 = 0x38, 2.0 = 0x40,
    # 3.0 = 0x44); W rows are one-hot: row 0 picks k = 0, row 1 picks k = 1,
    # row 2 picks k = 128. Per-row, per-block exponents: row 0 block 0: +1,
    # row 1 block 0: -2, row 2 block 1: +3, the rest 0, and activation
    # exponent 0: Q = [1 * 2, 2 * 2^-2, 3 * 8] = [2, 0.5, 24] (exact).
    a = np.zeros((1, 256), np.uint8)
    a[0, 0], a[0, 1], a[0, 128] = 0x38, 0x40, 0x44
    w = np.zeros((128, 256), np.uint8)
    w[0, 0] = w[1, 1] = w[2, 128] = 0x38
    sw = np.full((128, 2), 127, np.uint8)
    sw[0, 0], sw[1, 0], sw[2, 1] = 128, 125, 130
    sa = np.full((1, 2), 127, np.uint8)
    q = IQ.block_scaled_gemm(a, sa, w, sw)
    assert q[0, :3].tolist() == [2.0, 0.5, 24.0] and not np.any(q[0, 3:])
    # rows of a 128-row group sharing one exponent reduce to the per-tile layout
    g = np.random.default_rng(41)
    a2 = rand_codes(g, (3, 256))
    w2 = rand_codes(g, (256, 256))
    tile = g.integers(115, 130, size=(2, 2)).astype(np.uint8)
    sa2 = g.integers(120, 130, size=(3, 2)).astype(np.uint8)
    assert np.array_equal(IQ.block_scaled_gemm(a2, sa2, w2, np.repeat(tile, 128, axis=0)),
                          IQ.block_scaled_gemm(a2, sa2, w2, tile))
    with pytest.raises(ValueError):
        IQ.block_scaled_gemm(a2, sa2, w2, np.full((3, 2), 127, np.uint8))


# ---------------------------------------------------------------- RoPE


def test_rope_golden_unit_vectors():
    gd = json.load(open(os.path.join(GOLDEN, "rope_hadamard_closed_forms.json")))["rope"]
    for case in gd["cases"]:
        x = np.zeros((1, 1, 128))
        x[0, 0, case["unit"]] = 1.0
        y = IQ.rope_half_split(x, np.array([gd["position"]]), gd["theta"], gd["rope_dim"])[0, 0]
        want = np.zeros(128)
        for i, v in case["out"]:
            want[i] = v
        assert np.allclose(y, want, rtol=0, atol=1e-15), case["note"]


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(5).standard_normal((3, 4, 128))
    assert np.array_equal(IQ.rope_half_split(x, np.zeros(3, np.int64)), x)


def test_rope_preserves_pair_norms_and_composes():
    g = np.random.default_rng(6)
    x = g.standard_normal((8, 2, 128))
    p1 = g.integers(0, 131072, 8)
    p2 = g.integers(0, 131072, 8)
    y = IQ.rope_half_split(x, p1)
    n_in = x[..., :32] ** 2 + x[..., 32:64] ** 2
    n_out = y[..., :32] ** 2 + y[..., 32:64] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-13, atol=0)
    assert np.array_equal(y[..., 64:], x[..., 64:])
    z = IQ.rope_half_split(y, p2)
    direct = IQ.rope_half_split(x, p1 + p2)
    assert np.allclose(z, direct, rtol=0, atol=1e-9)


def test_rope_pairs_are_half_split_not_interleaved():
    x = np.zeros((1, 1, 128))
    x[0, 0, 0] = 1.0
    y = IQ.rope_half_split(x, np.array([1]))[0, 0]
    assert y[1] == 0.0 and y[32] != 0.0


def test_rope_table_closed_form():
    t = IQ.rope_cos_sin_table(10000.0, 5, 64)
    assert t.shape == (5, 64)
    for p in range(5):
        for i in (0, 1, 16, 31):
            ang = p * 10000.0 ** (-2 * i / 64)
            assert abs(t[p, i] - math.cos(ang)) < 1e-15 and abs(t[p, 32 + i] - math.sin(ang)) < 1e-15


# ---------------------------------------------------------------- Hadamard


def test_hadamard_orthogonality_and_symmetry():
    H = IQ.hadamard_matrix(128)
    assert np.array_equal(H @ H.T, 128 * np.eye(128))
    assert np.array_equal(H, H.T)
    Hn = H / np.sqrt(128)
    assert np.allclose(Hn @ Hn, np.eye(128), atol=1e-14)


def test_hadamard_matches_sylvester_recursion_and_butterflies():
    S = np.array([[1.0]])
    while S.shape[0] < 128:
        S = np.block([[S, S], [S, -S]])
    assert np.array_equal(IQ.hadamard_matrix(128), S)
    # brute-force radix-2 butterflies on a small random vector
    y = np.random.default_rng(7).standard_normal(128)
    v = y.copy()
    h = 1
    while h < 128:
        for i in range(0, 128, 2 * h):
            for j in range(i, i + h):
                v[j], v[j + h] = v[j] + v[j + h], v[j] - v[j + h]
        h *= 2
    assert np.allclose(IQ.hadamard_rotate(y), v / np.sqrt(128), rtol=0, atol=1e-13)


def test_hadamard_golden_and_norm():
    gd = json.load(open(os.path.join(GOLDEN, "rope_hadamard_closed_forms.json")))["hadamard"]
    c = gd["inv_sqrt_n"]
    r = np.arange(128)
    pop = np.array([bin(i).count("1") for i in r])
    rules = [np.full(128, c), np.where(r % 2 == 0, 2 * c, 0.0), np.where(pop % 2 == 0, c, -c)]
    for case, want in zip(gd["cases"], rules):
        x = np.zeros(128)
        for i, v in case["input_nonzero"]:
            x[i] = v
        assert np.allclose(IQ.hadamard_rotate(x), want, rtol=0, atol=1e-15), case["rule"]
    y = np.random.default_rng(8).standard_normal((10, 128))
    assert np.allclose(np.linalg.norm(IQ.hadamard_rotate(y), axis=1), np.linalg.norm(y, axis=1), rtol=1e-14)


# ---------------------------------------------------------------- FP4


def test_fp4_golden_worked_example():
    gd = json.load(open(os.path.join(GOLDEN, "fp4_worked_example.json")))
    z = np.zeros(128)
    for base, entries in gd["z"].items():
        for i, v in entries:
            z[int(base) + i] = v
    packed, sb = IQ.fp4_quantize(z[None, :])
    assert sb[0].tolist() == gd["scale_bytes"]
    for base, vals in gd["packed"].items():
        b = int(base)
        assert packed[0, b:b + len(vals)].tolist() == vals


@pytest.mark.parametrize("k", [-15, -7, 0, 5, 20])
def test_fp4_scale_closed_form(k):
    z = np.zeros((3, 32))
    z[0, 3] = 6.0 * 2.0 ** k
    z[1, 3] = np.nextafter(np.float32(6.0 * 2.0 ** k), np.float32(np.inf))
    z[2, 3] = np.nextafter(6.0 * 2.0 ** k, np.inf)          # one float64 ulp above
    _, sb = IQ.fp4_quantize(z)
    assert sb[0, 0] == 127 + k and sb[1, 0] == 128 + k and sb[2, 0] == 128 + k


def test_fp4_floor():
    z = np.zeros((3, 32))
    z[1, 0] = 1e-9
    z[2, 0] = -6.0 * 2.0 ** -15
    _, sb = IQ.fp4_quantize(z)
    assert sb[:, 0].tolist() == [112, 112, 112]


def test_fp4_dequant_error_bound():
    g = np.random.default_rng(9)
    z = g.standard_normal((50, 128)) * np.exp(g.uniform(-10, 10, (50, 1)))
    packed, sb = IQ.fp4_quantize(z)
    codes = F.e2m1_unpack(packed)
    scale = np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32, axis=1)
    deq = F.e2m1_decode(codes) * scale
    t = np.abs(z) / scale
    step = np.where(t < 2, 0.5, np.where(t < 4, 1.0, 2.0))
    assert np.all(np.abs(deq - z) <= step / 2 * scale)


def test_fp4_decision_is_taken_on_the_float64_value():
    """A float64 value a hair above a midpoint (one that float32 would round
    onto the midpoint) is decided on its exact value by default: it rounds
    up; rounded to float32 first it is a tie and goes to the even code."""
    z = np.zeros((1, 32))
    z[0, 0] = 6.0
    z[0, 1] = 0.25 + 2.0 ** -40
    packed, _ = IQ.fp4_quantize(z)
    assert F.e2m1_unpack(packed)[0, 1] == 1
    packed32, _ = IQ.fp4_quantize(z, decide_dtype=np.float32)
    assert F.e2m1_unpack(packed32)[0, 1] == 0
    # the same at a scale boundary: amax / 6 a hair above 2^0 takes e = 1 in
    # float64, e = 0 once rounded to float32
    z[0, 0] = 6.0 * (1.0 + 2.0 ** -40)
    _, sb = IQ.fp4_quantize(z)
    _, sb32 = IQ.fp4_quantize(z, decide_dtype=np.float32)
    assert sb[0, 0] == 128 and sb32[0, 0] == 127


# ---------------------------------------------------------------- chain


def test_chain_composes_the_stages():
    g = np.random.default_rng(10)
    M, K, H = 4, 256, 2
    a = rand_codes(g, (M, K))
    w = rand_codes(g, (H * 128, K))
    sa = g.integers(115, 130, size=(M, 2)).astype(np.uint8)
    sw = g.integers(110, 120, size=(H, 2)).astype(np.uint8)
    pos = g.integers(0, 4096, M)
    out = IQ.indexer_q_chain(a, sa, w, sw, pos, n_heads=H)
    q = IQ.block_scaled_gemm(a, sa, w, sw).reshape(M, H, 128)
    assert np.array_equal(out["q"], q)
    z = IQ.hadamard_rotate(IQ.rope_half_split(q, pos))
    assert np.array_equal(out["z"], z)
    p, s = IQ.fp4_quantize(z)
    assert np.array_equal(out["q_fp4"], p) and np.array_equal(out["q_scales"], s)
    assert out["q_fp4"].shape == (M, H, 64) and out["q_scales"].shape == (M, H, 4)


def test_chain_variants_closed_form():
    # A = e_0 (E4M3 1.0 = 0x38) and W row 0 = e_0, unit scales: Q = e_0 for
    # head 0 and 0 for head 1. At position 1 the interleaved pair (0, 1) turns
    # by 1 rad: z_r = (cos 1 + (-1)^bit0(r) sin 1) / sqrt(128), 0.12213 at even
    # r and -0.02662 at odd r. Ceil rule: e = -5 (byte 122), codes 4 (0x6) and
    # -1 (0xA), bytes 0xA6. OCP floor: e = -6 (byte 121), 7.82 saturates to 6
    # (0x7), -1.704 -> -1.5 (0xB), bytes 0xB7. Head 1 is all zero: floor
    # exponents -15 (ceil) and -16 (OCP floor), codes 0.
    K, H = 128, 2
    a = np.zeros((1, K), dtype=np.uint8)
    a[0, 0] = 0x38
    w = np.zeros((H * 128, K), dtype=np.uint8)
    w[0, 0] = 0x38
    sa = np.full((1, 1), 127, dtype=np.uint8)
    sw = np.full((H, 1), 127, dtype=np.uint8)
    pos = np.array([1])
    for rule, byte, code in (("ceil", 122, 0xA6), ("ocp_floor", 121, 0xB7)):
        out = IQ.indexer_q_chain(a, sa, w, sw, pos, n_heads=H, rope_layout="interleaved", scale_rule=rule)
        assert out["q_scales"][0, 0].tolist() == [byte] * 4
        assert out["q_fp4"][0, 0].tolist() == [code] * 64
        assert out["q_scales"][0, 1].tolist() == [127 + (-15 if rule == "ceil" else -16)] * 4
        assert out["q_fp4"][0, 1].tolist() == [0] * 64
    # the default layout at the same input: pair (0, 32), so dim 32 carries
    # sin 1 and the codes differ from the interleaved ones
    base = IQ.indexer_q_chain(a, sa, w, sw, pos, n_heads=H)
    assert not np.array_equal(base["q_fp4"][0, 0], np.full(64, 0xA6, dtype=np.uint8))


# ----------------------------------------------------------------------------
# Standalone epilogue (bf16 Q in): hand-derived closed forms
# ----------------------------------------------------------------------------


def _one_hot_q(d, value=1.0, n_heads=1):
    q = np.zeros((1, n_heads * 128))
    q[0, d] = value
    return q


def test_epilogue_pass_through_dim_gives_hadamard_column():
    # dim 69 >= 64 is not rotated; z = column 69 of H / sqrt(128), every entry
    # +-1/sqrt(128) = +-0.0884. amax/6 = 0.01473 lies in (2^-7, 2^-6]: e = -6,
    # byte 121; 0.0884 * 64 = 5.657 is above the 4|6 midpoint 5 -> magnitude 6,
    # code 7; the sign is (-1)^popcount(r & 69).
    out = IQ.indexer_q_epilogue(_one_hot_q(69), np.array([1234]), n_heads=1)
    assert out["q_scales"].tolist() == [[[121, 121, 121, 121]]]
    codes = F.e2m1_unpack(out["q_fp4"].reshape(-1))
    want = [7 | (8 if bin(r & 69).count("1") % 2 else 0) for r in range(128)]
    assert codes.tolist() == want


def test_epilogue_rotated_dim0_at_position_one():
    # dim 0 at position 1 rotates by 1 rad into (cos 1, sin 1) on dims (0, 32).
    # z_r = (cos 1 + (-1)^bit5(r) sin 1) / sqrt(128): 0.12213 where bit 5 of r
    # is clear, -0.02662 where it is set.
    #   blocks 0, 2: 0.12213/6 in (2^-6, 2^-5]: e = -5, byte 122; 0.12213*32 = 3.908
    #                is above the 3|4 midpoint 3.5 -> 4, code 6 -> bytes 0x66
    #   blocks 1, 3: 0.02662/6 in (2^-8, 2^-7]: e = -7, byte 120; 0.02662*128 = 3.407
    #                is below 3.5 -> 3, code 5, negative -> 0xD -> bytes 0xDD
    hi = (math.cos(1) + math.sin(1)) / math.sqrt(128)
    lo = (math.cos(1) - math.sin(1)) / math.sqrt(128)
    assert abs(hi * 32 - 3.5) > 0.3 and abs(abs(lo) * 128 - 3.5) > 0.05   # far from a boundary
    out = IQ.indexer_q_epilogue(_one_hot_q(0), np.array([1]), n_heads=1)
    assert out["q_scales"].tolist() == [[[122, 120, 122, 120]]]
    assert out["q_fp4"].reshape(-1).tolist() == [0x66] * 16 + [0xDD] * 16 + [0x66] * 16 + [0xDD] * 16


def test_epilogue_frequency_index_of_pair_16():
    # dim 16 at position 1000: angle 1000 * 10000^(-32/64) = 10 rad, into dims
    # (16, 48). z_r = (-1)^bit4(r) (cos 10 + (-1)^bit5(r) sin 10) / sqrt(128):
    #   bit 5 clear: |z| = 0.12225, sign -(-1)^bit4 -> e = -5 (byte 122),
    #                0.12225*32 = 3.912 -> 4, code 6: 0xE for r%32 < 16, 0x6 above
    #   bit 5 set:   |z| = 0.02608, sign -(-1)^bit4 -> e = -7 (byte 120),
    #                0.02608*128 = 3.338 -> 3, code 5: 0xD for r%32 < 16, 0x5 above
    a = abs(math.cos(10) + math.sin(10)) / math.sqrt(128)
    b = abs(math.cos(10) - math.sin(10)) / math.sqrt(128)
    assert abs(a * 32 - 3.5) > 0.3 and abs(b * 128 - 3.5) > 0.1
    out = IQ.indexer_q_epilogue(_one_hot_q(16), np.array([1000]), n_heads=1)
    assert out["q_scales"].tolist() == [[[122, 120, 122, 120]]]
    blk_hi = [0xEE] * 8 + [0x66] * 8
    blk_lo = [0xDD] * 8 + [0x55] * 8
    assert out["q_fp4"].reshape(-1).tolist() == blk_hi + blk_lo + blk_hi + blk_lo


def test_epilogue_heads_are_independent_and_match_the_chain_stages():
    rng = np.random.default_rng(7)
    M, H = 5, 3
    q = rng.standard_normal((M, H * 128))
    pos = rng.integers(0, 4096, M)
    out = IQ.indexer_q_epilogue(q, pos, n_heads=H)
    for h in range(H):
        one = IQ.indexer_q_epilogue(q[:, 128 * h:128 * (h + 1)], pos, n_heads=1)
        assert np.array_equal(one["q_fp4"][:, 0], out["q_fp4"][:, h])
        assert np.array_equal(one["q_scales"][:, 0], out["q_scales"][:, h])
    # rotation and Hadamard preserve each head's norm
    np.testing.assert_allclose(np.linalg.norm(out["z"], axis=-1),
                               np.linalg.norm(q.reshape(M, H, 128), axis=-1), rtol=1e-13)


# ----------------------------------------------------------------------------
# Convention variants: interleaved RoPE pairs, OCP floor-rule FP4 scales
# ----------------------------------------------------------------------------


def test_rope_interleaved_closed_forms_and_invariants():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((3, 2, 128))
    pos = np.array([0, 5, 4000])
    out = IQ.rope_interleaved(q, pos)
    assert np.array_equal(out[0], q[0])                       # position 0: identity
    assert np.array_equal(out[:, :, 64:], q[:, :, 64:])       # pass-through dims
    n_in = q[..., 0:64:2] ** 2 + q[..., 1:64:2] ** 2
    n_out = out[..., 0:64:2] ** 2 + out[..., 1:64:2] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13)       # pair norms
    # composition: rotating by p1 then p2 is rotating by p1 + p2
    two = IQ.rope_interleaved(IQ.rope_interleaved(q, np.array([7, 7, 7])), np.array([11, 11, 11]))
    np.testing.assert_allclose(two, IQ.rope_interleaved(q, np.array([18, 18, 18])), atol=1e-12)
    # e_32 (pair i = 16) at position 1000: angle 1000 * 10000^(-32/64) = 10 rad onto dims (32, 33)
    e = np.zeros((1, 1, 128))
    e[0, 0, 32] = 1.0
    r = IQ.rope_interleaved(e, np.array([1000]))
    assert abs(r[0, 0, 32] - math.cos(10)) < 1e-12 and abs(r[0, 0, 33] - math.sin(10)) < 1e-12
    assert np.count_nonzero(r) == 2
    # and it is not the half-split layout
    assert not np.allclose(r, IQ.rope_half_split(e, np.array([1000])))


def test_fp4_ocp_floor_rule_worked_example():
    # e = floor(log2 amax) - 2, codes saturate at 6:
    #   block 0: amax 6 = 1.5 * 2^2 -> e = 0 (byte 127); 6 -> 7; 5 -> tie 4|6 -> even code 6 (4);
    #            -0.25 -> tie 0|0.5 -> 0 (negative zero 8)
    #   block 1: amax 7 -> e = 0 (byte 127); 7 saturates to 6 (code 7); 3 -> 5
    #   block 2: amax 3.9 -> e = -1 (byte 126); 3.9 * 2 = 7.8 -> 6 (code 7); 1 * 2 = 2 -> 4
    #   block 3: amax 1e-5, floored to 1e-4 = 1.6384 * 2^-14 -> e = -16 (byte 111);
    #            1e-5 * 2^16 = 0.655 -> below the 0.5|1 midpoint 0.75 -> 0.5 (code 1)
    z = np.zeros(128)
    z[0], z[1], z[2] = 6.0, 5.0, -0.25
    z[32], z[33] = 7.0, 3.0
    z[64], z[65] = 3.9, 1.0
    z[96] = 1e-5
    packed, sb = IQ.fp4_quantize(z, scale_rule="ocp_floor")
    assert sb.tolist() == [127, 127, 126, 111]
    codes = F.e2m1_unpack(packed).tolist()
    assert codes[0:3] == [7, 6, 8] and codes[32:34] == [7, 5] and codes[64:66] == [7, 4] and codes[96] == 1
    # the default rule on the same block 1 never saturates: e = 1, 7/2 = 3.5 -> tie 3|4 -> 4 (code 6)
    packed_c, sb_c = IQ.fp4_quantize(z)
    assert sb_c[1] == 128 and F.e2m1_unpack(packed_c)[32] == 6


def test_epilogue_variants_closed_forms():
    # dim 0 at position 1, interleaved: (cos 1, sin 1) on dims (0, 1), so
    # z_r = (cos 1 + (-1)^bit0(r) sin 1) / sqrt(128): 0.12213 at even r,
    # -0.02662 at odd r, in every block.
    #   ceil rule: e = -5 (byte 122); 3.908 -> 4 (code 6), -0.852 -> above the
    #   0.5|1 midpoint -> -1 (code 0xA): bytes 0xA6
    #   OCP floor: 0.12213 = 1.954 * 2^-4 -> e = -6 (byte 121); 7.82 -> 6 (code 7),
    #   -1.704 -> below the 1.5|2 midpoint -> -1.5 (code 0xB): bytes 0xB7
    q = np.zeros((1, 128))
    q[0, 0] = 1.0
    out = IQ.indexer_q_epilogue(q, np.array([1]), n_heads=1, rope_layout="interleaved")
    assert out["q_scales"].tolist() == [[[122] * 4]] and out["q_fp4"].reshape(-1).tolist() == [0xA6] * 64
    out = IQ.indexer_q_epilogue(q, np.array([1]), n_heads=1, rope_layout="interleaved", scale_rule="ocp_floor")
    assert out["q_scales"].tolist() == [[[121] * 4]] and out["q_fp4"].reshape(-1).tolist() == [0xB7] * 64


# ----------------------------------------------------------------------------
# Explicit frequency schedules (a table of any frequencies, YaRN-style scaling)
# ----------------------------------------------------------------------------


def test_rope_explicit_frequencies_closed_forms():
    # inv_freq[0] = 0.5 at position 2: pair 0 turns by exactly 1 rad; mscale
    # 1.25 scales cos and sin. Half-split puts the pair on dims (0, 32),
    # interleaved on dims (0, 1).
    inv = np.zeros(32)
    inv[0] = 0.5
    e = np.zeros((1, 1, 128))
    e[0, 0, 0] = 1.0
    hs = IQ.rope_half_split(e, np.array([2]), inv_freq=inv, mscale=1.25)
    assert abs(hs[0, 0, 0] - 1.25 * math.cos(1)) < 1e-15 and abs(hs[0, 0, 32] - 1.25 * math.sin(1)) < 1e-15
    assert np.count_nonzero(hs) == 2
    il = IQ.rope_interleaved(e, np.array([2]), inv_freq=inv, mscale=1.25)
    assert abs(il[0, 0, 0] - 1.25 * math.cos(1)) < 1e-15 and abs(il[0, 0, 1] - 1.25 * math.sin(1)) < 1e-15
    assert np.count_nonzero(il) == 2
    # a zero frequency leaves its pair alone at any position (mscale 1)
    rng = np.random.default_rng(31)
    q = rng.standard_normal((2, 3, 128))
    out = IQ.rope_half_split(q, np.array([5, 77]), inv_freq=np.zeros(32))
    assert np.array_equal(out, q)
    # mscale scales the rotated dims' norm and leaves the pass-through dims
    out = IQ.rope_half_split(q, np.array([5, 77]), inv_freq=np.linspace(0.0, 1.0, 32), mscale=0.5)
    np.testing.assert_allclose(np.linalg.norm(out[..., :64], axis=-1), 0.5 * np.linalg.norm(q[..., :64], axis=-1),
                               rtol=1e-13)
    assert np.array_equal(out[..., 64:], q[..., 64:])
    with pytest.raises(ValueError):
        IQ.rope_angles(np.array([1]), 10000.0, 64, inv_freq=np.ones(31))
