"""Pins of the oracle's fp64 matmul.

Definition (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical
Formulation"; ternary case with zero bias): y[m,n] = sum_g s[n,g] *
sum_j x[m, gG+j] * c[n, gG+j].  The references here decode the packed bytes
with numpy.base_repr (not the oracle's decoder) and sum in exact rationals or
with numpy.matmul.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs


def decode_independent(packed, N, K, G):
    B = (G + 4) // 5
    p = packed.reshape(N, K // G, B)
    lut = np.array([[int(ch) - 1 for ch in reversed(np.base_repr(v, 3).zfill(5))] for v in range(243)], np.int8)
    codes = lut[p].reshape(N, K // G, 5 * B)[:, :, :G]
    return codes.reshape(N, K)


@pytest.mark.parametrize("N,K,G,M", [(3, 320, 64, 2), (8, 640, 128, 3), (5, 70, 7, 1), (2, 64, 64, 3)])
def test_matmul_vs_exact_rationals(N, K, G, M):
    w = inputs.normal_bf16(21, (N, K), 0.02)
    x = inputs.activation(22, M, K)
    packed, scales, _ = oracle.quantize_pack(w, G)
    y, bound, st = oracle.matmul(x, packed, scales, N, K, G)
    assert st == 0
    codes = decode_independent(packed, N, K, G)
    s = [[Fraction(float(v)) for v in row] for row in scales.view(np.float16)]
    xf = [[Fraction(float(v)) for v in row] for row in inputs.bf16_bits_to_f32(x)]
    for m in range(M):
        for n in range(N):
            exact = sum((xf[m][k] * int(codes[n, k]) * s[n][k // G] for k in range(K)), Fraction(0))
            b = sum((abs(xf[m][k] * int(codes[n, k]) * s[n][k // G]) for k in range(K)), Fraction(0))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 10 ** 12) * b + Fraction(0)
            assert abs(Fraction(bound[m, n]) - b) <= Fraction(1, 10 ** 12) * b


def test_matmul_vs_numpy_matmul():
    N, K, G, M = 64, 1024, 128, 4
    w = inputs.normal_bf16(23, (N, K), 0.02)
    x = inputs.activation(24, M, K)
    packed, scales, _ = oracle.quantize_pack(w, G)
    y, bound, _ = oracle.matmul(x, packed, scales, N, K, G)
    What = decode_independent(packed, N, K, G).astype(np.float64) * np.repeat(
        scales.view(np.float16).astype(np.float64), G, axis=1)
    xf = inputs.bf16_bits_to_f32(x).astype(np.float64)
    ref = xf @ What.T
    assert np.all(np.abs(y - ref) <= 1e-12 * bound)
    assert np.allclose(bound, np.abs(xf) @ np.abs(What).T, rtol=1e-12, atol=0)


def test_one_hot_rows_exact():
    N, K, G = 16, 256, 64
    w = inputs.normal_bf16(25, (N, K), 0.02)
    packed, scales, _ = oracle.quantize_pack(w, G)
    codes = decode_independent(packed, N, K, G)
    ks = [0, 1, 4, 5, 63, 64, 129, 255]
    x = np.zeros((len(ks), K), np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80  # 1.0
    y, _, _ = oracle.matmul(x, packed, scales, N, K, G)
    s = scales.view(np.float16).astype(np.float64)
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], codes[:, k] * s[:, k // G])


def test_invalid_byte_in_matmul_flagged():
    N, K, G = 4, 128, 64
    w = inputs.normal_bf16(26, (N, K), 0.02)
    packed, scales, _ = oracle.quantize_pack(w, G)
    p = packed.copy()
    p[2, 3] = 250
    x = inputs.activation(27, 1, K)
    _, _, st = oracle.matmul(x, p, scales, N, K, G)
    assert st & oracle.INVALID_BYTE
