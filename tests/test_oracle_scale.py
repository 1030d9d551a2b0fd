"""Pins of the oracle's group scale and codes.

Rule (precisit "pack-unpack-run" README, codec.py description and scale-rule
paragraph): the mean of |w| over a group, rounded to fp16; nearest-even
ternary codes.  Reading: the sum is exact and rounded once (round half to
even); code = +-1 iff |w| > s/2, ties to 0.

The reference used here is independent of the oracle's integer arithmetic:
exact rational means (fractions.Fraction) rounded by brute force over the
table of all finite fp16 values, numpy's float64 -> float16 conversion where
the mean is exact in float64, and numpy's round-half-even rint for the codes.
"""
import bisect
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs

_TABLE = None


def fp16_table():
    global _TABLE
    if _TABLE is None:
        vals = [Fraction(float(v)) for v in np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)]
        vals.append(Fraction(65536))  # stands for the overflow bits 0x7C00
        _TABLE = vals
    return _TABLE


def rne_fp16_bits(q: Fraction) -> int:
    """Nearest fp16 bits of q >= 0 by table search; ties to even bits."""
    t = fp16_table()
    if q >= t[-1]:
        return 0x7C00
    i = bisect.bisect_right(t, q) - 1
    if t[i] == q:
        return i
    d_lo, d_hi = q - t[i], t[i + 1] - q
    if d_lo != d_hi:
        return i if d_lo < d_hi else i + 1
    return i if i % 2 == 0 else i + 1


def frac_bf16(b) -> Fraction:
    return Fraction(float(inputs.bf16_bits_to_f32(np.array([b], np.uint16))[0]))


def ref_scale_bits(group) -> int:
    q = sum((abs(frac_bf16(b)) for b in group), Fraction(0)) / len(group)
    return rne_fp16_bits(q)


def random_finite_bf16(rng, n, emin=0, emax=254):
    sign = rng.integers(0, 2, n).astype(np.uint16) << 15
    e = rng.integers(emin, emax + 1, n).astype(np.uint16) << 7
    m = rng.integers(0, 128, n).astype(np.uint16)
    return sign | e | m


def check_groups(w, G):
    packed, scales, st = oracle.quantize_pack(w, G)
    for r in range(w.shape[0]):
        for g in range(w.shape[1] // G):
            want = ref_scale_bits(w[r, g * G:(g + 1) * G])
            assert int(scales[r, g]) == want, (r, g, hex(int(scales[r, g])), hex(want))
    return packed, scales, st


@pytest.mark.parametrize("G", [64, 128, 5, 7, 100])
def test_scale_vs_fraction_normal(G):
    w = inputs.normal_bf16(11, (40, 4 * G), 0.02)
    check_groups(w, G)


@pytest.mark.parametrize("G", [64, 128])
def test_scale_vs_fraction_wide_exponents(G):
    rng = np.random.default_rng(12)
    # exponents spread over the whole range below the fp16 overflow region,
    # so exact sums span up to ~140 binades (subnormal bf16 included)
    w = random_finite_bf16(rng, 60 * G, 0, 140).reshape(60, G)
    check_groups(w, G)
    # narrow bands near the fp16 subnormal / underflow boundary
    w = random_finite_bf16(rng, 60 * G, 95, 115).reshape(60, G)
    check_groups(w, G)


def test_scale_overflow_and_underflow():
    G = 64
    big = np.full((1, G), inputs.f32_to_bf16_bits(np.array([7e4], np.float32))[0], np.uint16)
    packed, scales, st = oracle.quantize_pack(big, G)
    assert st & oracle.SCALE_OVERFLOW and scales[0, 0] == 0x7C00
    assert (packed == 121).all()
    tiny = np.full((1, G), inputs.f32_to_bf16_bits(np.array([2.0 ** -30], np.float32))[0], np.uint16)
    packed, scales, st = oracle.quantize_pack(tiny, G)
    assert st == 0 and scales[0, 0] == 0
    # mean exactly 65504 (largest finite) is fine; 65520 rounds to overflow
    w = np.zeros((2, 64), np.uint16)
    w[0, :] = inputs.f32_to_bf16_bits(np.array([65504.0], np.float32))[0]  # bf16(65504) = 65536
    assert ref_scale_bits(w[0]) == 0x7C00


def test_nonfinite_flagged():
    w = inputs.normal_bf16(13, (2, 64), 0.02)
    w[1, 5] = 0x7F80  # +inf
    packed, scales, st = oracle.quantize_pack(w, 64)
    assert st & oracle.NONFINITE
    assert scales[1, 0] == 0x7E00 and (packed[1] == 121).all()


def test_scale_closed_forms_numpy():
    rng = np.random.default_rng(14)
    vals = random_finite_bf16(rng, 400, 100, 140)
    for b in vals:
        v = float(inputs.bf16_bits_to_f32(np.array([b & 0x7FFF], np.uint16))[0])
        w = np.full((1, 64), b, np.uint16)
        _, s_all, st = oracle.quantize_pack(w, 64)
        want = np.array([v], np.float64).astype(np.float16).view(np.uint16)[0]
        if want >= 0x7C00:
            assert st & oracle.SCALE_OVERFLOW
        else:
            assert s_all[0, 0] == want
        w1 = np.zeros((1, 64), np.uint16)
        w1[0, 17] = b
        _, s_one, _ = oracle.quantize_pack(w1, 64)
        assert s_one[0, 0] == np.array([v / 64], np.float64).astype(np.float16).view(np.uint16)[0]


def test_scale_library_pin_fsum():
    """Where math.fsum of a group is exact, numpy's float16(fsum/G) must agree."""
    w = inputs.normal_bf16(15, (200, 128), 0.02)
    for G in (64, 128):
        _, scales, _ = oracle.quantize_pack(w, G)
        f = inputs.bf16_bits_to_f32(w).astype(np.float64)
        for r in range(w.shape[0]):
            for g in range(128 // G):
                grp = np.abs(f[r, g * G:(g + 1) * G])
                s = math.fsum(grp)
                if Fraction(s) == sum((Fraction(float(v)) for v in grp), Fraction(0)):
                    assert scales[r, g] == np.array([s / G]).astype(np.float16).view(np.uint16)[0]


def _bf16(v):
    return int(inputs.f32_to_bf16_bits(np.array([v], np.float32))[0])


def test_scale_constructed_midpoints():
    """Exact means on fp16 midpoints round to even; a 2^-100 excess rounds up."""
    G = 64
    cases = [
        # 63 x 1.0 + 1 x (1 + 2^-5): mean 1 + 2^-11, midpoint of 0x3C00/0x3C01 -> 0x3C00
        ([1.0] * 63 + [1.0 + 2.0 ** -5], 0x3C00),
        # mean 1 + 3*2^-11: midpoint of 0x3C01/0x3C02 -> 0x3C02
        ([1.0] * 63 + [1.0 + 3 * 2.0 ** -5], 0x3C02),
    ]
    for vals, want in cases:
        w = np.array([[_bf16(v) for v in vals]], np.uint16)
        _, s, st = oracle.quantize_pack(w, G)
        assert st == 0 and s[0, 0] == want, (hex(int(s[0, 0])), hex(want))
    # A midpoint plus 2^-100: an fp32 or fp64 running sum would drop the tail
    # and round to even; the exact sum lies above the midpoint and rounds up.
    G = 128
    vals = [2.0] * 63 + [2.0 + 2.0 ** -4] + [2.0 ** -100] + [0.0] * 63
    w = np.array([[_bf16(v) for v in vals]], np.uint16)
    _, s, st = oracle.quantize_pack(w, G)
    # exact mean = (128 + 2^-4 + 2^-100)/128 = 1 + 2^-11 + 2^-107 -> 0x3C01
    assert s[0, 0] == 0x3C01
    assert ref_scale_bits(w[0]) == 0x3C01
    vals[64] = 0.0
    w = np.array([[_bf16(v) for v in vals]], np.uint16)
    _, s, _ = oracle.quantize_pack(w, G)
    assert s[0, 0] == 0x3C00  # exact tie -> even


def test_codes_tie_fixture():
    """32 x +-1.5 and 32 x +-0.5: s = 1.0; |w| = s/2 is a tie that goes to 0."""
    rng = np.random.default_rng(16)
    mags = np.array([1.5] * 32 + [0.5] * 32, np.float32)
    rng.shuffle(mags)
    signs = rng.choice([-1.0, 1.0], 64).astype(np.float32)
    w = inputs.f32_to_bf16_bits(mags * signs)[None, :]
    packed, scales, st = oracle.quantize_pack(w, 64)
    assert scales[0, 0] == 0x3C00
    codes, _ = oracle.unpack(packed, 1, 64, 64)
    want = np.where(mags == 1.5, signs, 0).astype(np.int8)
    assert np.array_equal(codes[0], want)


def test_codes_vs_numpy_rint():
    """For s > 0, codes equal clip(rint(w/s), -1, 1) with numpy's float32
    division and round-half-even rint."""
    w = np.concatenate([inputs.normal_bf16(17, (300, 128), 0.02),
                        random_finite_bf16(np.random.default_rng(18), 300 * 128, 100, 135).reshape(300, 128)])
    for G in (64, 128):
        packed, scales, st = oracle.quantize_pack(w, G)
        codes, _ = oracle.unpack(packed, w.shape[0], 128, G)
        s32 = np.repeat(scales.view(np.float16).astype(np.float32), G, axis=1)
        w32 = inputs.bf16_bits_to_f32(w)
        ok = s32 > 0
        ref = np.clip(np.rint(w32[ok] / s32[ok]), -1, 1).astype(np.int8)
        assert np.array_equal(codes[ok], ref)
        # s == 0 (underflow): sign codes by the literal rule
        assert np.array_equal(codes[~ok], np.sign(w32[~ok]).astype(np.int8))
