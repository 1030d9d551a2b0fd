"""Pins of the oracle's QAT forward (fake quantization): w_hat =
bf16_RNE(c * s) with the group scale and code rule of the precisit
"pack-unpack-run" README (codec.py description, scale-rule paragraph) and
the BitNet-style training of the Avenue README.

Expected values come from exact rationals written here: the mean of |w| as a
Fraction rounded to the nearest fp16 (ties to even), codes from comparing
|w| with s/2 exactly, and the nearest bf16 of c * s."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.test_oracle_dequantize import f16_value, nearest_bf16
from tests.test_oracle_scale import frac_bf16, random_finite_bf16, ref_scale_bits


def ref_group(group):
    sbits = ref_scale_bits(group)
    s = f16_value(sbits)
    out = []
    for b in group:
        v = frac_bf16(int(b))
        c = 1 if v > s / 2 else (-1 if v < -s / 2 else 0)
        out.append(nearest_bf16(c * s, negative_zero=(c == -1) != bool(sbits & 0x8000)))
    return sbits, out


@pytest.mark.parametrize("G", [64, 128, 5])
def test_random_groups_match_exact_definition(G):
    rng = np.random.default_rng(400 + G)
    N, K = 6, 4 * G
    w = random_finite_bf16(rng, N * K, emin=100, emax=140).reshape(N, K)
    w_hat, sc, st = oracle.fake_quantize(w, G)
    assert st == 0
    for r in range(N):
        for g in range(K // G):
            sbits, want = ref_group(w[r, g * G:(g + 1) * G])
            assert int(sc[r, g]) == sbits
            assert [int(v) for v in w_hat[r, g * G:(g + 1) * G]] == want, (r, g)


def test_ties_and_saturation_written_out():
    """A group with mean 1: +-0.5 (= s/2) are ties and go to code 0, whose
    value 0 * s is +0 whatever the weight's sign; 1.5 and 2.5 saturate at
    code 1; -0.75 and -1.25 give -1."""
    vals = [0.5, -0.5, 1.5, 2.5, -0.75, 0.0, 1.0, -1.0] + [1.0] * 56
    vals[7] = -(64 - sum(abs(v) for v in vals[:7]) - 56)   # mean |w| exactly 1
    g = np.array(vals, np.float32)
    assert abs(g).sum() == 64
    bits = (g.view(np.uint32) >> 16).astype(np.uint16)     # all exact in bf16
    w_hat, sc, st = oracle.fake_quantize(bits.reshape(1, 64), 64)
    assert st == 0 and int(sc[0, 0]) == 0x3C00
    got = [int(v) for v in w_hat[0, :8]]
    assert got == [0x0000, 0x0000, 0x3F80, 0x3F80, 0xBF80, 0x0000, 0x3F80, 0xBF80]


def test_flagged_groups_are_zero():
    G = 64
    w = np.full((3, 2 * G), 0x3C00, np.uint16)             # bf16 0.0078125
    w[0, 5] = 0x7FC0                                       # NaN in group (0, 0)
    w[1, G:] = 0x7F00                                      # 2^127: mean overflows fp16
    w_hat, sc, st = oracle.fake_quantize(w, G)
    assert st == 1 | 2
    assert (w_hat[0, :G] == 0).all() and int(sc[0, 0]) == 0x7E00
    assert (w_hat[1, G:] == 0).all() and int(sc[1, 1]) == 0x7C00
    sbits, want = ref_group(w[2, :G])
    assert [int(v) for v in w_hat[2, :G]] == want
    assert (w_hat[0, G:] == w_hat[2, :G]).all()


def test_consistent_with_pack_then_decode():
    """On unflagged data, the fused forward equals packing followed by the
    decode (both oracle functions; the pins above fix each separately)."""
    from ternary_weight_only_amd import inputs
    w = inputs.normal_bf16(410, (40, 640), 0.02)
    for G in (64, 128):
        w_hat, sc, st = oracle.fake_quantize(w, G)
        p, s, st2 = oracle.quantize_pack(w, G)
        d, st3 = oracle.dequantize(p, s, 40, 640, G)
        assert st == st2 == st3 == 0
        assert np.array_equal(sc, s) and np.array_equal(w_hat, d)
