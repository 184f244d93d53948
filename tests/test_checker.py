"""Self-tests for the acceptance rules: planted differences on the CPU must be
accepted exactly when they are legal rounding-boundary flips."""
import numpy as np
import pytest

from oracle import checker as C
from oracle import formats as F
from oracle import indexer_q as IQ


def make_case(seed=0, rows=64):
    g = np.random.default_rng(seed)
    z = g.standard_normal((rows, 2, 128))
    packed, sb = IQ.fp4_quantize(z)
    return z, packed, sb


def set_code(packed, idx, code):
    p = packed.copy()
    m, h, e = idx
    byte = p[m, h, e // 2]
    if e % 2 == 0:
        p[m, h, e // 2] = (byte & 0xF0) | code
    else:
        p[m, h, e // 2] = (byte & 0x0F) | (code << 4)
    return p


def test_identical_passes():
    z, p, s = make_case()
    r = C.check_fp4(p, s, z, p, s)
    assert r["ok"] and r["code_mismatch"] == 0 and r["rel_l2"] == 0


def test_boundary_flip_accepted_interior_flip_rejected():
    z, p, s = make_case()
    # put a value exactly on the 1.25 midpoint (codes 2|3) in block 0 of (0, 0)
    scale = np.ldexp(1.0, int(s[0, 0, 0]) - 127)
    z = z.copy()
    z[0, 0, 5] = 1.25 * scale
    p, s = IQ.fp4_quantize(z)
    assert F.e2m1_unpack(p)[0, 0, 5] == 2
    ok = C.check_fp4(set_code(p, (0, 0, 5), 3), s, z, p, s)
    assert ok["ok"] and ok["code_mismatch"] == 1 and ok["code_illegal"] == 0
    # a flip of an element far from any midpoint is illegal
    codes = F.e2m1_unpack(p)
    sc = z / np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    frac_dist = np.abs(np.abs(sc) - np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])[:, None, None, None]).min(axis=0)
    m, h, e = np.argwhere((frac_dist > 0.1) & (codes % 8 > 0) & (codes % 8 < 7))[0]
    c = int(codes[m, h, e])
    bad = C.check_fp4(set_code(p, (m, h, e), c + 1), s, z, p, s)
    assert not bad["ok"] and bad["code_illegal"] == 1


def test_two_step_flip_rejected():
    z, p, s = make_case(1)
    scale = np.ldexp(1.0, int(s[3, 1, 2]) - 127)
    z = z.copy()
    z[3, 1, 70] = 2.5 * scale
    p, s = IQ.fp4_quantize(z)
    assert F.e2m1_unpack(p)[3, 1, 70] == 4
    bad = C.check_fp4(set_code(p, (3, 1, 70), 6), s, z, p, s)
    assert not bad["ok"]


def test_signed_zero_is_not_a_difference():
    z, p, s = make_case(2)
    codes = F.e2m1_unpack(p)
    m, h, e = np.argwhere(codes == 0)[0]
    r = C.check_fp4(set_code(p, (m, h, e), 8), s, z, p, s)
    assert r["ok"] and r["code_mismatch"] == 0


def test_scale_flip_only_at_power_of_two_boundary():
    z, p, s = make_case(3, rows=256)      # 2048 blocks: one flip is under 0.1 %
    z = z.copy()
    # block (5, 0, 1): make amax exactly 6 * 2^k so amax/6 is a power of two
    blk = z[5, 0, 32:64]
    i = int(np.argmax(np.abs(blk)))
    k = 2
    z[5, 0, 32 + i] = np.sign(blk[i]) * 6.0 * 2.0 ** k
    z[5, 0, 32:64] = np.clip(z[5, 0, 32:64], -6.0 * 2 ** k, 6.0 * 2 ** k)
    p, s = IQ.fp4_quantize(z)
    assert s[5, 0, 1] == 127 + k
    # the device rounded the amax up by an ulp: scale one higher, codes at that scale
    s_dev = s.copy()
    s_dev[5, 0, 1] += 1
    blkz = z[5, 0, 32:64] * 2.0 ** -(k + 1)
    p_dev = p.copy()
    codes = F.e2m1_unpack(p_dev)
    codes[5, 0, 32:64] = F.e2m1_encode_rne(blkz)
    p_dev = F.e2m1_pack(codes)
    r = C.check_fp4(p_dev, s_dev, z, p, s)
    assert r["scale_mismatch"] == 1 and r["scale_illegal"] == 0 and r["code_illegal"] == 0 and r["ok"]
    # the same flip on a block whose amax is far from a power of two is illegal
    s_bad = s.copy()
    blk = np.abs(z[7, 1, :32]).max() / 6
    assert abs(blk / 2.0 ** np.round(np.log2(blk)) - 1) > 0.01
    s_bad[7, 1, 0] += 1
    assert not C.check_fp4(p, s_bad, z, p, s)["ok"]


def test_too_many_boundary_flips_rejected():
    g = np.random.default_rng(4)
    z = g.standard_normal((100, 1, 128))
    p, s = IQ.fp4_quantize(z)
    scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    # place 2% of elements (none of them a block maximum) exactly on the 0.75
    # midpoint, then flip them all legally
    bmax = np.repeat(np.abs(z).reshape(100, 1, 4, 32).max(axis=-1), 32, axis=-1)
    idx = np.argwhere(np.abs(z) < 0.5 * bmax)[::20]
    assert len(idx) > 0.02 * z.size
    z2 = z.copy()
    for m, h, e in idx:
        z2[m, h, e] = 0.75 * scale[m, h, e]
    p2, s2 = IQ.fp4_quantize(z2)
    assert np.array_equal(s2, s)
    pd = p2
    for m, h, e in idx:
        pd = set_code(pd, (m, h, e), 1)      # 0.5 instead of 1.0: the other side of the tie
    r = C.check_fp4(pd, s2, z2, p2, s2)
    assert r["code_illegal"] == 0 and not r["ok"]


def test_rel_l2_fails_on_wrong_output():
    z, p, s = make_case(5)
    z2, p2, s2 = make_case(6)
    r = C.check_fp4(p2, s2, z, p, s)
    assert not r["ok"] and r["rel_l2"] > 0.5


def test_fp8_check():
    q = np.arange(256, dtype=np.uint8).reshape(2, 128)
    s = np.array([[1], [2]], dtype=np.int32)
    assert C.check_fp8_quant(q, s, q, s)["ok"]
    q2 = q.copy()
    q2[1, 3] ^= 1
    r = C.check_fp8_quant(q2, s, q, s)
    assert not r["ok"] and r["q_mismatch"] == 1
    with pytest.raises(ValueError):
        C.check_fp8_quant(q[:1], s, q, s)


def test_one_boundary_flip_allowed_in_a_small_sample_two_are_not():
    """256 blocks (one token, 64 heads): 0.1 % of them is below one, so one
    legal scale flip passes and two do not."""
    z, p, s = make_case(5, rows=32)          # 32 x 2 x 4 = 256 blocks
    z = z.copy()
    flips = []
    for m, h, b in ((3, 0, 1), (9, 1, 2)):
        blk = z[m, h, 32 * b:32 * b + 32]
        i = int(np.argmax(np.abs(blk)))
        z[m, h, 32 * b + i] = np.sign(blk[i]) * 6.0                 # amax / 6 exactly 2^0
        z[m, h, 32 * b:32 * b + 32] = np.clip(z[m, h, 32 * b:32 * b + 32], -6.0, 6.0)
        flips.append((m, h, b))
    p, s = IQ.fp4_quantize(z)

    def flipped(n):
        s_dev = s.copy()
        codes = F.e2m1_unpack(p)
        for m, h, b in flips[:n]:
            s_dev[m, h, b] += 1
            codes[m, h, 32 * b:32 * b + 32] = F.e2m1_encode_rne(z[m, h, 32 * b:32 * b + 32] * 0.5)
        return F.e2m1_pack(codes), s_dev

    p1, s1 = flipped(1)
    r1 = C.check_fp4(p1, s1, z, p, s)
    assert r1["blocks"] == 256 and r1["scale_mismatch"] == 1 and r1["scale_illegal"] == 0 and r1["ok"]
    p2, s2 = flipped(2)
    r2 = C.check_fp4(p2, s2, z, p, s)
    assert r2["scale_mismatch"] == 2 and r2["scale_illegal"] == 0 and not r2["ok"]


# ---------------------------------------------------------------- OCP floor rule
#
# Under scale_rule="ocp_floor" the exponent is floor(log2 amax) - 2: it steps
# where amax itself (equivalently amax / 4) crosses a power of two, not where
# amax / 6 does, and codes saturate at +-6.


def _floor_block(amax, rows=64, seed=11):
    """rows x 2 heads x 128 dims of N(0, (amax/4)^2) whose block (0, 0, 0)
    has the given amax (its other elements kept below it)."""
    z = np.random.default_rng(seed).standard_normal((rows, 2, 128)) * (amax / 4)
    blk = np.clip(z[0, 0, :32], -0.9 * amax, 0.9 * amax)
    blk[7] = amax
    z[0, 0, :32] = blk
    return z


def _requantize_block(p, s, z, e_dev):
    """Device output whose block (0, 0, 0) uses exponent e_dev with codes
    rounded at that scale (saturating at +-6)."""
    s_dev = s.copy()
    s_dev[0, 0, 0] = 127 + e_dev
    codes = F.e2m1_unpack(p)
    codes[0, 0, :32] = F.e2m1_encode_rne(np.clip(z[0, 0, :32] * 2.0 ** -e_dev, -6.0, 6.0))
    return F.e2m1_pack(codes), s_dev


@pytest.mark.parametrize("k", [-3, 0, 4])
def test_floor_rule_scale_flip_legal_within_window_of_a_power_of_two(k):
    # amax just below 2^(k+2): the oracle's exponent is k - 1; a device that
    # rounded amax up onto 2^(k+2) takes k. amax / 4 is within 2^-10 of 2^k.
    amax = 2.0 ** (k + 2) * (1 - 2.0 ** -12)
    z = _floor_block(amax)
    p, s = IQ.fp4_quantize(z, scale_rule="ocp_floor")
    assert s[0, 0, 0] == 127 + k - 1
    p_dev, s_dev = _requantize_block(p, s, z, k)
    r = C.check_fp4(p_dev, s_dev, z, p, s, scale_rule="ocp_floor")
    assert r["scale_mismatch"] == 1 and r["scale_illegal"] == 0 and r["code_illegal"] == 0 and r["ok"], r
    # the ceil rule's window (amax / 6 near a power of two) does not cover it
    r_ceil = C.check_fp4(p_dev, s_dev, z, p, s)
    assert r_ceil["scale_illegal"] == 1 and not r_ceil["ok"]
    # and a flip in the other direction (amax just above 2^(k+2)) is legal too
    amax = 2.0 ** (k + 2) * (1 + 2.0 ** -12)
    z = _floor_block(amax)
    p, s = IQ.fp4_quantize(z, scale_rule="ocp_floor")
    assert s[0, 0, 0] == 127 + k
    p_dev, s_dev = _requantize_block(p, s, z, k - 1)
    r = C.check_fp4(p_dev, s_dev, z, p, s, scale_rule="ocp_floor")
    assert r["scale_mismatch"] == 1 and r["scale_illegal"] == 0 and r["code_illegal"] == 0 and r["ok"], r


def test_floor_rule_scale_flip_just_outside_the_window_is_illegal():
    amax = 4.0 * (1 - 2.0 ** -9)          # amax / 4 is 2^-9 away from 2^0
    z = _floor_block(amax)
    p, s = IQ.fp4_quantize(z, scale_rule="ocp_floor")
    assert s[0, 0, 0] == 126
    p_dev, s_dev = _requantize_block(p, s, z, 0)
    r = C.check_fp4(p_dev, s_dev, z, p, s, scale_rule="ocp_floor")
    assert r["scale_illegal"] == 1 and not r["ok"]


def test_floor_rule_flip_at_a_ceil_boundary_is_illegal():
    # amax / 6 = 2^0 exactly: a legal flip under the ceil rule, but under the
    # floor rule amax = 6 is far (6 / 4 = 1.5) from any power of two
    z = _floor_block(6.0)
    p, s = IQ.fp4_quantize(z, scale_rule="ocp_floor")
    assert s[0, 0, 0] == 127
    p_dev, s_dev = _requantize_block(p, s, z, 1)
    r = C.check_fp4(p_dev, s_dev, z, p, s, scale_rule="ocp_floor")
    assert r["scale_illegal"] == 1 and not r["ok"]


def test_floor_rule_saturated_codes():
    # amax 7.5 * 2^-1 -> e = floor(log2 3.75) - 2 = -1; the element scales to
    # 7.5 and saturates to 6 (code 7); its negative twin to code 0xF
    z = _floor_block(3.75)
    z[0, 0, 9] = -3.75
    p, s = IQ.fp4_quantize(z, scale_rule="ocp_floor")
    assert s[0, 0, 0] == 126
    codes = F.e2m1_unpack(p)
    assert codes[0, 0, 7] == 7 and codes[0, 0, 9] == 15
    assert C.check_fp4(p, s, z, p, s, scale_rule="ocp_floor")["ok"]
    # a device that wrote 4 (code 6) for the saturated 6 is wrong: 7.5 is not
    # within the window of the 4|6 midpoint
    bad = C.check_fp4(set_code(p, (0, 0, 7), 6), s, z, p, s, scale_rule="ocp_floor")
    assert bad["code_illegal"] == 1 and not bad["ok"]
    bad = C.check_fp4(set_code(p, (0, 0, 9), 14), s, z, p, s, scale_rule="ocp_floor")
    assert bad["code_illegal"] == 1 and not bad["ok"]


def test_floor_rule_code_flip_only_at_a_midpoint():
    z = _floor_block(3.75)
    z[0, 0, 3] = 2.5 * 0.5                 # scaled 2.5: the 2|3 midpoint
    z[0, 0, 4] = 2.2 * 0.5                 # scaled 2.2: interior
    p, s = IQ.fp4_quantize(z, scale_rule="ocp_floor")
    codes = F.e2m1_unpack(p)
    assert codes[0, 0, 3] == 4 and codes[0, 0, 4] == 4      # 2.5 ties to even code 4 (2.0)
    ok = C.check_fp4(set_code(p, (0, 0, 3), 5), s, z, p, s, scale_rule="ocp_floor")
    assert ok["code_mismatch"] == 1 and ok["code_illegal"] == 0 and ok["ok"]
    bad = C.check_fp4(set_code(p, (0, 0, 4), 5), s, z, p, s, scale_rule="ocp_floor")
    assert bad["code_illegal"] == 1 and not bad["ok"]


def test_floor_rule_floor_byte():
    # amax below 1e-4 = 1.6384 * 2^-14: exponent -16 (byte 111) on both sides
    z = _floor_block(3e-5)
    z[0, 0, :32] *= 1e-4
    z[0, 0, 7] = 3e-5
    p, s = IQ.fp4_quantize(z, scale_rule="ocp_floor")
    assert s[0, 0, 0] == 111
    assert C.check_fp4(p, s, z, p, s, scale_rule="ocp_floor")["ok"]
