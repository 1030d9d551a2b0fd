"""Pins of the W4A16 oracle (tiny-llm "Week 2 Day 3: Quantize the Model":
"Group-Wise Affine Quantization", "Reconstruct a Stored Group", "Packed
Storage Layout", "Mathematical Formulation", "Computation Flow").

The oracle's matmul takes the page's per-element order (reconstruct q*s + b,
multiply by the activation, add).  The pins check it against the page's
printed layout and orientation example, against the page's factored form
s * sum(x q) + b * sum(x) written out in numpy from an independent unpack,
and against closed forms and invariants."""
import os

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fixture(golden=GOLDEN):
    words, orient = [], []
    for line in open(os.path.join(golden, "w4a16_layout_and_orientation.txt")):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "word":
            words.append((int(f[1], 16), [int(v) for v in f[2:]]))
        elif f[0] == "orient":
            orient.append(tuple(float(v) for v in f[1:]))
    return words, orient


def bf16(v):
    out = inputs.f32_to_bf16_bits(np.asarray(v, np.float32))
    return out.item() if np.ndim(v) == 0 else out


def bf16_val(bits):
    return inputs.bf16_bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def numpy_unpack(packed, N, K):
    """Independent unpack: shift each word by 4i for i = 0..7."""
    p = np.asarray(packed, np.uint64).reshape(N, K // 8)
    return ((p[:, :, None] >> (4 * np.arange(8, dtype=np.uint64))) & 0xF).reshape(N, K)


def random_problem(seed, N, K, G):
    return inputs.w4a16_problem(seed, N, K, G)


def test_packing_layout_fixture(golden=GOLDEN):
    words, _ = _fixture(golden)
    p = np.array([w for w, _ in words], np.uint32)
    codes = oracle.w4_unpack(p, len(words), 8)
    assert codes.tolist() == [c for _, c in words]


def test_orientation_example(golden=GOLDEN):
    """Both printed pairs: q = 0 and q = 15 reconstruct the printed values
    (the page says "about" for q = 15: bf16 storage moves 0.0867 by at most
    half an ulp, 2^-12, which q = 15 multiplies by 15, and 0.8 by at most
    2^-9, so under 0.005 in all), and the two pairs give the same endpoints
    in opposite order."""
    _, orient = _fixture(golden)
    G = K = 128
    ends = []
    for s, b, at0, at15 in orient:
        packed = np.zeros((1, K // 8), np.uint32)
        packed[0, 0] = 0xF0                     # weight 0: q = 0; weight 1: q = 15
        w = oracle.w4a16_dequantize(packed, bf16([[s]]), bf16([[b]]), 1, K, G)
        assert abs(w[0, 0] - at0) < 0.005 and abs(w[0, 1] - at15) < 0.005
        assert (w[0, 2:] == w[0, 0]).all()
        ends.append((w[0, 0], w[0, 1]))
    (a0, a15), (b0, b15) = ends
    assert abs(a0 - b15) < 0.01 and abs(a15 - b0) < 0.01


def test_one_hot_rows_equal_reconstructed_weights():
    N, K, G = 9, 256, 128
    packed, s, b = random_problem(1, N, K, G)
    w = oracle.w4a16_dequantize(packed, s, b, N, K, G)
    for k in (0, 7, 8, 127, 128, 255):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = bf16(1.0)
        y, _ = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
        assert np.array_equal(y[0], w[:, k]), k


@pytest.mark.parametrize("N,K,G,M", [(3, 128, 128, 1), (17, 1024, 128, 2), (5, 512, 64, 3),
                                     (4, 384, 128, 1)])
def test_matmul_vs_factored_form(N, K, G, M):
    """The page's rearranged sum: per group s * sum_j x_j q_j + b * sum_j x_j,
    from the numpy unpack, in fp64."""
    packed, s, b = random_problem(10 + N, N, K, G)
    x = inputs.activation(20 + K, M, K)
    y, bound = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
    q = numpy_unpack(packed, N, K).astype(np.float64)
    xf = bf16_val(x)
    sf, bf = bf16_val(s), bf16_val(b)
    nG = K // G
    yf = np.zeros((M, N))
    for g in range(nG):
        xs = xf[:, g * G:(g + 1) * G]
        yf += sf[:, g][None, :] * (xs @ q[:, g * G:(g + 1) * G].T) + bf[:, g][None, :] * xs.sum(1)[:, None]
    assert (np.abs(y - yf) <= 1e-12 * bound).all()
    # bound written out from its terms
    bd = np.abs(xf) @ (np.abs(q * np.repeat(sf, G, axis=1)) + np.abs(np.repeat(bf, G, axis=1))).T
    assert np.allclose(bound, bd, rtol=1e-12, atol=0)


def test_codes_only_reduce_to_integer_matmul():
    """s = 1, b = 0: y = x @ q^T, an exact fp64 numpy matmul of small
    integers against bf16 activations."""
    N, K, G = 6, 256, 64
    packed, _, _ = random_problem(3, N, K, G)
    s = np.full((N, K // G), bf16(1.0), np.uint16)
    b = np.zeros((N, K // G), np.uint16)
    x = inputs.activation(4, 2, K)
    y, _ = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
    q = numpy_unpack(packed, N, K).astype(np.float64)
    assert np.allclose(y, bf16_val(x) @ q.T, rtol=1e-13, atol=0)


def test_bias_only():
    """All codes 0: y = sum_g b_g * sum_{j in g} x_j."""
    N, K, G = 5, 512, 128
    _, s, b = random_problem(5, N, K, G)
    packed = np.zeros((N, K // 8), np.uint32)
    x = inputs.activation(6, 1, K)
    y, bound = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
    xs = bf16_val(x)[0].reshape(K // G, G).sum(1)
    assert np.allclose(y[0], bf16_val(b) @ xs, rtol=1e-12, atol=0)


def test_nonnegative_terms_bound_equals_y():
    N, K, G = 7, 256, 128
    packed, s, b = random_problem(7, N, K, G)
    s = bf16(np.abs(bf16_val(s)))
    b = bf16(np.abs(bf16_val(b)))
    x = bf16(np.abs(bf16_val(inputs.activation(8, 2, K))))
    y, bound = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
    assert np.allclose(y, bound, rtol=1e-13, atol=0)


def test_orientation_flip_gives_same_result():
    """(q, s, b) and (15 - q, -s, b + 15 s) reconstruct the same weights (the
    page's two orientations); with s and b on a grid of 2^-6 every value is
    exact, so the results are identical."""
    N, K, G = 6, 256, 128
    rng = np.random.default_rng(9)
    packed, _, _ = random_problem(9, N, K, G)
    sv = rng.integers(1, 16, size=(N, K // G)) / 64.0
    bv = rng.integers(-64, 0, size=(N, K // G)) / 64.0
    flipped = (~packed).astype(np.uint32)         # every nibble q -> 15 - q
    x = inputs.activation(10, 1, K)
    y1, _ = oracle.w4a16_matmul(x, packed, bf16(sv), bf16(bv), N, K, G)
    y2, _ = oracle.w4a16_matmul(x, flipped, bf16(-sv), bf16(bv + 15 * sv), N, K, G)
    assert np.array_equal(y1, y2)


def test_shape_errors():
    p = np.zeros((1, 16), np.uint32)
    s = np.zeros((1, 1), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.w4a16_matmul(np.zeros((1, 128), np.uint16), p, s, s, 1, 128, 96)
    with pytest.raises(oracle.OracleError):
        oracle.w4a16_dequantize(p, s, s, 1, 128, 4)
