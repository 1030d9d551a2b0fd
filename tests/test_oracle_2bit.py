"""Pins of the oracle's 2-bit ternary format (Avenue README, size note:
2-bit packing; "Autoregressive Language Model on the 6502 Processor": four
ternary parameters a byte), against the base-3 path, which its own pins fix,
and exhaustive checks of the byte code."""
import itertools

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs


@pytest.mark.parametrize("G", [64, 128, 4, 12])
def test_codes_and_scales_agree_with_the_base3_format(G):
    w = inputs.normal_bf16(900 + G, (24, 4 * G if G >= 64 else 96), 0.02)
    N, K = w.shape
    p2, s2, st2 = oracle.quantize_pack2(w, G)
    c2, u2 = oracle.unpack2(p2, N, K, G)
    p3, s3, st3 = oracle.quantize_pack(w, G)
    c3, _ = oracle.unpack(p3, N, K, G)
    assert st2 == st3 == 0 and u2 == 0
    assert p2.shape == (N, K // 4)
    assert np.array_equal(s2, s3)
    assert np.array_equal(c2, c3)


def test_byte_code_is_a_bijection_with_the_first_weight_lowest():
    """All 81 four-code combinations: distinct bytes, each field 0..2, the
    first weight in bits 0-1, and unpack2 gives the codes back."""
    seen = set()
    for codes in itertools.product((-1, 0, 1), repeat=4):
        # a group of 4 weights with these codes: |w| = 1.5 for +-1, 0 for 0
        vals = np.array([1.5 * c for c in codes] + [1.5] * 4, np.float32)
        bits = (vals.view(np.uint32) >> 16).astype(np.uint16).reshape(1, 8)
        p, s, st = oracle.quantize_pack2(bits, 8)
        c, _ = oracle.unpack2(p, 1, 8, 8)
        assert st == 0 and list(c[0, :4]) == list(codes)
        b = int(p[0, 0])
        assert all(((b >> (2 * i)) & 3) != 3 for i in range(4))
        assert (b & 3) == codes[0] + 1
        seen.add(b)
    assert len(seen) == 81


def test_field_three_is_flagged_and_reads_as_zero():
    p = np.array([[0b11_10_01_00, 0b01_01_01_01]], np.uint8)
    c, st = oracle.unpack2(p, 1, 8, 8)
    assert st == oracle.INVALID_BYTE
    assert list(c[0]) == [-1, 0, 1, 0, 0, 0, 0, 0]


def test_matmul2_equals_the_base3_matmul_of_the_same_weights():
    rng_x = inputs.activation(905, 3, 256)
    w = inputs.normal_bf16(906, (40, 256), 0.02)
    for G in (64, 128):
        p2, s2, _ = oracle.quantize_pack2(w, G)
        p3, s3, _ = oracle.quantize_pack(w, G)
        y2, b2, st2 = oracle.matmul2(rng_x, p2, s2, 40, 256, G)
        y3, b3, st3 = oracle.matmul(rng_x, p3, s3, 40, 256, G)
        assert st2 == st3 == 0
        assert np.array_equal(y2, y3) and np.array_equal(b2, b3)
