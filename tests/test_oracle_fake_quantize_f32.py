"""Pins of the oracle's QAT forward from fp32 latent weights: w_hat = c * s in
fp32 (exact), with the group scale and code rule of the precisit
"pack-unpack-run" README (codec.py description, scale-rule paragraph) applied
to the fp32 weights themselves (Avenue README, introduction: BitNet-style
training keeps full-precision latent weights).

Expected values come from exact rationals written here: the mean of |w| as a
Fraction rounded to the nearest fp16 (ties to even, by table search), codes
from comparing w with s/2 exactly, and c * s, which fp32 holds exactly."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.test_oracle_dequantize import f16_value
from tests.test_oracle_scale import rne_fp16_bits


def f32(v) -> np.float32:
    return np.float32(v)


def ref_group_f32(group):
    """(scale bits, status, expected w_hat float32 list) of one fp32 group."""
    vals = [Fraction(float(v)) for v in group]
    if not all(np.isfinite(group)):
        return 0x7E00, 1, [f32(0.0)] * len(group)
    q = sum((abs(v) for v in vals), Fraction(0)) / len(group)
    sbits = rne_fp16_bits(q)
    if sbits >= 0x7C00:
        return 0x7C00, 2, [f32(0.0)] * len(group)
    s = f16_value(sbits)
    out = []
    for v in vals:
        c = 1 if v > s / 2 else (-1 if v < -s / 2 else 0)
        if s == 0:
            out.append(f32(-0.0) if c == -1 else f32(0.0))
        else:
            out.append(f32(float(c * s)))
    return sbits, 0, out


def check_exact(w, G):
    w_hat, sc, st = oracle.fake_quantize_f32(w, G)
    st_all = 0
    for r in range(w.shape[0]):
        for g in range(w.shape[1] // G):
            grp = w[r, g * G:(g + 1) * G]
            sbits, gst, want = ref_group_f32(grp)
            st_all |= gst
            assert int(sc[r, g]) == sbits, (r, g, hex(int(sc[r, g])), hex(sbits))
            got = w_hat[r, g * G:(g + 1) * G]
            assert got.view(np.uint32).tolist() == np.array(want, np.float32).view(
                np.uint32).tolist(), (r, g)
    assert st == st_all
    return w_hat, sc


@pytest.mark.parametrize("G", [64, 128, 5])
def test_normal_groups_match_exact_definition(G):
    rng = np.random.default_rng(800 + G)
    w = (rng.standard_normal((6, 4 * G)) * 0.02).astype(np.float32)
    check_exact(w, G)


@pytest.mark.parametrize("G", [64, 128])
def test_wide_exponents_match_exact_definition(G):
    """Random finite fp32 bit patterns over exponents -149 .. +15, subnormals
    included, so the exact sum spans far more than 64 bits."""
    rng = np.random.default_rng(810 + G)
    n = 8 * 2 * G
    sign = rng.integers(0, 2, n).astype(np.uint32) << 31
    e = rng.integers(0, 142, n).astype(np.uint32) << 23
    m = rng.integers(0, 1 << 23, n).astype(np.uint32)
    w = (sign | e | m).view(np.float32).reshape(8, 2 * G)
    check_exact(w, G)


def test_scale_uses_the_fp32_values():
    """Weights 1 + 2^-11 (not representable in bf16, which would round them
    to 1): a group of them has its mean on the midpoint between the fp16
    values 1 and 1 + 2^-10 and rounds to even (1.0); one extra 2^-20 on one
    weight puts the mean above the midpoint (1 + 2^-10)."""
    G = 64
    base = f32(1.0 + 2.0 ** -11)
    tie = np.full(G, base, np.float32)
    up = tie.copy()
    up[17] = f32(1.0 + 2.0 ** -11 + 2.0 ** -20)
    _, sc, st = oracle.fake_quantize_f32(np.stack([tie, up]), G)
    assert st == 0
    assert int(sc[0, 0]) == 0x3C00 and int(sc[1, 0]) == 0x3C01


def test_code_ties_at_fp32_resolution():
    """With s = 1: |w| = 0.5 exactly is a tie (code 0, w_hat +0); one fp32
    step above 0.5 gives +-1; 1.5 saturates at 1."""
    G = 64
    half_up = np.nextafter(f32(0.5), f32(1.0))
    vals = [0.5, -0.5, half_up, -half_up, 1.5, -1.5, 0.0, 1.0]
    # |vals| sum to 6 + 2^-23; 54 ones, 2 - 2^-23 and 2 make the total 64
    w = np.array(vals + [1.0] * 54 + [2.0 - 2.0 ** -23, 2.0], np.float32)
    assert sum(Fraction(float(abs(v))) for v in w) == G
    w_hat, sc, st = oracle.fake_quantize_f32(w.reshape(1, G), G)
    assert st == 0 and int(sc[0, 0]) == 0x3C00
    assert w_hat[0, :8].tolist() == [0.0, 0.0, 1.0, -1.0, 1.0, -1.0, 0.0, 1.0]
    assert not np.signbit(w_hat[0, 1])                     # code 0 of a negative weight: +0


def test_flags_and_underflow():
    """NaN or Inf: NONFINITE, scale 0x7E00, w_hat +0.  A mean above the fp16
    range: SCALE_OVERFLOW, 0x7C00, +0.  A mean below 2^-25: s = +0, codes by
    the rule (|w| > 0 gives +-1), w_hat the signed zero c * (+0)."""
    G = 64
    w = np.tile(np.array([0.01, -0.01], np.float32), (4, G // 2))
    w[0, 3] = np.float32(np.nan)
    w[1, 9] = np.float32(np.inf)
    w[2, :] = np.tile(np.array([3.0e38, -3.0e38], np.float32), G // 2)
    w[3, :] = np.array([1e-40, -1e-40] * (G // 2), np.float32)   # subnormals
    w_hat, sc, st = oracle.fake_quantize_f32(w, G)
    assert st == 1 | 2
    assert int(sc[0, 0]) == 0x7E00 and int(sc[1, 0]) == 0x7E00 and int(sc[2, 0]) == 0x7C00
    for r in range(3):
        assert (w_hat[r].view(np.uint32) == 0).all()
    assert int(sc[3, 0]) == 0
    assert w_hat[3].view(np.uint32).tolist() == [0x00000000, 0x80000000] * (G // 2)


def test_agrees_with_bf16_forward_on_bf16_values():
    """On weights exactly representable in bf16, the fp32 forward has the same
    scales as the bf16 forward, and its w_hat rounded to bf16 is the bf16
    forward's w_hat (both oracle functions; each is pinned on its own)."""
    from ternary_weight_only_amd import inputs
    wb = inputs.normal_bf16(820, (20, 640), 0.02)
    w = inputs.bf16_bits_to_f32(wb).astype(np.float32)
    for G in (64, 128):
        h32, s32, st32 = oracle.fake_quantize_f32(w, G)
        h16, s16, st16 = oracle.fake_quantize(wb, G)
        assert st32 == st16 == 0 and np.array_equal(s32, s16)
        assert np.array_equal(inputs.f32_to_bf16_bits(h32), h16)
