"""GPU parity of the W4A16 decode GEMV (tq_w4a16_gemv, tq_w4a16_gemv_batched)
against the CPU oracle (tiny-llm "Week 2 Day 3: Quantize the Model":
"Group-Wise Affine Quantization", "Packed Storage Layout", "Mathematical
Formulation", "Computation Flow").

Bar: the kernel's fp32 sum lies within 1e-3 * sum_k |x| (|q s| + |b|) of the
oracle's fp64 sum, and its one rounding to bf16 adds at most half a bf16 ulp,
which is at most 2^-8 of the value rounded:
    |y - y_ref| <= 1e-3 * B * (1 + 2^-8) + 2^-8 * |y_ref|."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import dev_bf16, host_u16, say
from tests.test_oracle_w4a16 import bf16, random_problem

pytestmark = pytest.mark.gpu


def dev_u32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).to("cuda")


def gpu_w4(x, packed, s, b, N, K, G):
    import torch
    import ternary_weight_only_amd as tq
    y = tq.w4a16_gemv(dev_bf16(x), dev_u32(packed), dev_bf16(s), dev_bf16(b), N, K, G)
    torch.cuda.synchronize()
    return host_u16(y)[0]


def bf16_val(bits):
    return inputs.bf16_bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def check(y_bits, y_ref, bound, what):
    y = bf16_val(y_bits)
    tol = 1e-3 * bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y_ref)
    bad = ~(np.abs(y - y_ref) <= tol)
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError("%s: %d of %d outside the bar; first at %d: gpu=%r ref=%r tol=%r"
                             % (what, int(bad.sum()), bad.size, i, y[i], y_ref[i], tol[i]))


@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (3, 128, 128), (17, 640, 64), (250, 1024, 128),
                                   (1025, 1088, 64), (100, 2048, 128), (300, 2112, 64),
                                   (64, 4096, 128), (3584, 1024, 128), (1024, 3584, 128),
                                   (70001, 256, 64)])
def test_w4a16_gemv_parity(N, K, G):
    """Both scale orientations in every matrix; ragged ring rounds and
    partial row steps; every lanes-per-row width; a grid at its cap."""
    packed, s, b = random_problem(400 + N, N, K, G)
    x = inputs.activation(401 + K, 1, K)
    say("w4a16 W[%d,%d] G=%d" % (N, K, G))
    y = gpu_w4(x, packed, s, b, N, K, G)
    y_ref, bound = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
    check(y, y_ref[0], bound[0], "W[%d,%d] G=%d" % (N, K, G))


@pytest.mark.parametrize("G", [64, 128])
def test_w4a16_one_hot_exact(G):
    """x = e_k: the kernel's value is fp32(q s + b) (q s is exact in fp32),
    rounded once to bf16."""
    N, K = 300, 1024
    packed, s, b = random_problem(410, N, K, G)
    w = oracle.w4a16_dequantize(packed, s, b, N, K, G)
    for k in (0, 63, 64, G - 1, G + 9, K - 1):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = bf16(1.0)
        y = gpu_w4(x, packed, s, b, N, K, G)
        expect = inputs.f32_to_bf16_bits(w[:, k].astype(np.float32))
        assert np.array_equal(y, expect), k


def test_w4a16_bias_only_and_codes_only():
    N, K, G = 512, 1024, 128
    packed, s, b = random_problem(420, N, K, G)
    x = inputs.activation(421, 1, K)
    zero = np.zeros_like(packed)
    y = gpu_w4(x, zero, s, b, N, K, G)
    y_ref, bound = oracle.w4a16_matmul(x, zero, s, b, N, K, G)
    check(y, y_ref[0], bound[0], "bias only")
    nob = np.zeros_like(b)
    y = gpu_w4(x, packed, s, nob, N, K, G)
    y_ref, bound = oracle.w4a16_matmul(x, packed, s, nob, N, K, G)
    check(y, y_ref[0], bound[0], "codes only")


def test_w4a16_batched_matches_single_bitwise_at_stack_shapes():
    import torch
    import ternary_weight_only_amd as tq
    G = 128
    for N, K, count in ((3584, 1024, 5), (1024, 3584, 3)):
        probs = [random_problem(430 + i + K, N, K, G) for i in range(count)]
        xs = [inputs.activation(440 + i + K, 1, K) for i in range(count)]
        say("w4a16 batched %d x W[%d,%d]" % (count, N, K))
        ys = tq.w4a16_gemv_batched([dev_bf16(x) for x in xs], [dev_u32(p) for p, _, _ in probs],
                                   [dev_bf16(s) for _, s, _ in probs],
                                   [dev_bf16(b) for _, _, b in probs], N, K, G)
        torch.cuda.synchronize()
        for i, (p, s, b) in enumerate(probs):
            yb = host_u16(ys[i])[0]
            assert np.array_equal(yb, gpu_w4(xs[i], p, s, b, N, K, G)), i
            y_ref, bound = oracle.w4a16_matmul(xs[i], p, s, b, N, K, G)
            check(yb, y_ref[0], bound[0], "batched %d" % i)


def test_w4a16_repeatable():
    N, K, G = 3584, 1024, 128
    packed, s, b = random_problem(450, N, K, G)
    x = inputs.activation(451, 1, K)
    assert np.array_equal(gpu_w4(x, packed, s, b, N, K, G), gpu_w4(x, packed, s, b, N, K, G))


def test_w4a16_nonfinite_scale_propagates_to_its_row_only():
    """A NaN or Inf group scale reaches y of its own row only (q * NaN is
    NaN; q * Inf is Inf, or NaN where q = 0); every other row stays within
    the bar."""
    N, K, G = 64, 512, 128
    packed, s, b = random_problem(460, N, K, G)
    x = inputs.activation(461, 1, K)
    s = s.copy()
    s[5, 1] = 0x7FC0                              # NaN
    s[40, 3] = 0x7F80                             # +Inf
    y = bf16_val(gpu_w4(x, packed, s, b, N, K, G))
    assert np.isnan(y[5]) and not np.isfinite(y[40])
    keep = np.ones(N, bool)
    keep[[5, 40]] = False
    y_ref, bound = oracle.w4a16_matmul(x, packed[keep], s[keep], b[keep], int(keep.sum()), K, G)
    tol = 1e-3 * bound[0] * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y_ref[0])
    assert (np.abs(y[keep] - y_ref[0]) <= tol).all()


def test_w4a16_grouped_mixed_shapes_bitwise_equal_to_single():
    """One grouped launch over problems of different shapes (the stack's two,
    a single row, ragged and long rows, both G's lane widths): each result
    bit-identical to tq_w4a16_gemv alone and within the bar."""
    import torch
    import ternary_weight_only_amd as tq
    G = 128
    shapes = [(3584, 1024)] * 4 + [(1024, 3584)] * 3 + [(1, 128), (777, 2048), (64, 4096),
                                                        (300, 1152)]
    probs = [random_problem(600 + i, N, K, G) for i, (N, K) in enumerate(shapes)]
    xs = [inputs.activation(620 + i, 1, K) for i, (N, K) in enumerate(shapes)]
    say("w4a16 grouped %d problems" % len(shapes))
    ys = tq.w4a16_gemv_grouped([dev_bf16(x) for x in xs], [dev_u32(p) for p, _, _ in probs],
                               [dev_bf16(s) for _, s, _ in probs], [dev_bf16(b) for _, _, b in probs],
                               [N for N, _ in shapes], [K for _, K in shapes], G)
    torch.cuda.synchronize()
    for i, ((N, K), (p, s, b)) in enumerate(zip(shapes, probs)):
        yg = host_u16(ys[i])[0]
        assert np.array_equal(yg, gpu_w4(xs[i], p, s, b, N, K, G)), i
        y_ref, bound = oracle.w4a16_matmul(xs[i], p, s, b, N, K, G)
        check(yg, y_ref[0], bound[0], "grouped %d" % i)
