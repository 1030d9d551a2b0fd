"""Grouped decode GEMV (M = 1) at stack sizes: many problems of mixed shapes
in one tq_gemv_grouped call, against the CPU oracle: |y - y_ref| <=
1e-3 * sum_k |x_k w_hat_k| per element, one-hot activations bit-exact
(tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation").

The packed bytes are random valid bytes (padding trits included, which the
matmul ignores) with random fp16 scales; every output is checked against the oracle on the
same bytes."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import assert_within_bound, dev_bf16, dev_f16bits, dev_u8, say

pytestmark = pytest.mark.gpu


def _problem(rng, N, K, G):
    B = (G + 4) // 5
    p = rng.integers(0, 243, size=(N, (K // G) * B)).astype(np.uint8)
    s = (rng.uniform(0.002, 0.05, size=(N, K // G)).astype(np.float16)).view(np.uint16)
    return p, s


def _grouped(problems, xs, G):
    import torch
    import ternary_weight_only_amd as tq
    st = tq.new_status()
    pk = [dev_u8(p) for p, _ in problems]
    sc = [dev_f16bits(s) for _, s in problems]
    xd = [dev_bf16(x) for x in xs]
    Ns = [p.shape[0] for p, _ in problems]
    Ks = [x.shape[1] for x in xs]
    ys = tq.gemv_grouped(xd, pk, sc, Ns, Ks, G, status=st)
    torch.cuda.synchronize()
    return [y.cpu().numpy().reshape(-1) for y in ys], int(st.item())


def _check_rows(y, x, p, s, K, G, rows, what):
    y_ref, bound, _ = oracle.matmul(x, p[rows], s[rows], len(rows), K, G)
    assert_within_bound(y[rows].reshape(1, -1), y_ref, bound, what)


@pytest.mark.parametrize("G", [64, 128])
def test_ffn_stack_shapes_every_output(G):
    """48 x W[3584,1024] and 24 x W[1024,3584] in one grouped call (12288 row
    tiles), each with its own activations: every output of every problem."""
    rng = np.random.default_rng(800 + G)
    shapes = [(3584, 1024)] * 48 + [(1024, 3584)] * 24
    problems = [_problem(rng, N, K, G) for N, K in shapes]
    xs = [inputs.activation(810 + i, 1, K) for i, (N, K) in enumerate(shapes)]
    say("grouped gemv: FFN stack shapes G=%d" % G)
    ys, st = _grouped(problems, xs, G)
    assert st == 0
    for i, ((N, K), (p, s)) in enumerate(zip(shapes, problems)):
        _check_rows(ys[i], xs[i], p, s, K, G, np.arange(N), "problem %d W[%d,%d]" % (i, N, K))


@pytest.mark.parametrize("G", [64, 128])
def test_ragged_rows_mixed_k_invalid_bytes(G):
    """100 problems with N not a multiple of 16 and K from 1024 to 4160, every
    output of every problem checked, invalid bytes at the first and the very
    last byte of two problems flagged."""
    rng = np.random.default_rng(820 + G)
    Ks = [1024, 2048, 2560, 4096, 1088, 4160]
    shapes = [(1000 + 7 * (i % 5), Ks[i % len(Ks)] if Ks[i % len(Ks)] % G == 0 else 1024)
              for i in range(100)]
    problems = [_problem(rng, N, K, G) for N, K in shapes]
    xs = [inputs.activation(830 + i, 1, K) for i, (N, K) in enumerate(shapes)]
    say("grouped gemv: 100 ragged problems G=%d" % G)
    ys, st = _grouped(problems, xs, G)
    assert st == 0
    for i in range(100):
        N, K = shapes[i]
        _check_rows(ys[i], xs[i], problems[i][0], problems[i][1], K, G, np.arange(N),
                    "problem %d all rows" % i)
    for i, pos in ((5, (0, 0)), (99, (-1, -1))):   # the first and the very last byte
        bad = [(p.copy(), s) for p, s in problems]
        bad[i][0][pos] = 250 if i == 5 else 255
        _, st = _grouped(bad, xs, G)
        assert st == 4, (i, st)


def test_one_hot_activations_exact():
    """x = e_k: y[n] is s[n, k/G] * c[n, k], bit for bit."""
    G = 128
    rng = np.random.default_rng(840)
    shapes = [(3584, 1024)] * 20
    problems = [_problem(rng, N, K, G) for N, K in shapes]
    xs = []
    for i, (N, K) in enumerate(shapes):
        x = np.zeros((1, K), np.uint16)
        x[0, (37 * i + 5) % K] = 0x3F80   # 1.0
        xs.append(x)
    say("grouped gemv: one-hot")
    ys, st = _grouped(problems, xs, G)
    assert st == 0
    for i in range(20):
        N, K = shapes[i]
        y_ref, _, _ = oracle.matmul(xs[i], problems[i][0], problems[i][1], N, K, G)
        assert np.array_equal(ys[i], y_ref.reshape(-1).astype(np.float32)), i


def test_wide_range_activations():
    """Activations spanning 2^-60 .. 2^20 in one vector, and a problem whose
    nonzero codes meet only values below 2^-40: the bound is relative to
    sum |x w_hat| of each row, so the tiny products must come out right."""
    G = 64
    rng = np.random.default_rng(850)
    shapes = [(2048, 1024)] * 32
    problems = [_problem(rng, N, K, G) for N, K in shapes]
    xs = []
    for i, (N, K) in enumerate(shapes):
        e = rng.integers(-60, 21, size=K).astype(np.float64)
        v = (rng.choice([-1.0, 1.0], size=K) * np.exp2(e)).astype(np.float32)
        xs.append(inputs.f32_to_bf16_bits(v).reshape(1, K))
    # problem 0: codes are nonzero only where |x| < 2^-40
    p0, s0 = problems[0]
    tiny = np.abs(inputs.bf16_bits_to_f32(xs[0].reshape(-1))) < 2.0 ** -40
    codes = rng.integers(0, 3, size=(2048, 1024)) - 1
    codes[:, ~tiny] = 0
    B = (G + 4) // 5
    p0 = np.zeros_like(p0)
    for g in range(1024 // G):
        blk = np.concatenate([codes[:, g * G:(g + 1) * G] + 1,
                              np.ones((2048, 5 * B - G), np.int64)], axis=1)
        for b in range(B):
            p0[:, g * B + b] = (blk[:, 5 * b:5 * b + 5] * np.array([1, 3, 9, 27, 81])).sum(1)
    problems[0] = (p0, s0)
    say("grouped gemv: wide-range activations")
    ys, st = _grouped(problems, xs, G)
    assert st == 0
    for i in range(32):
        N, K = shapes[i]
        _check_rows(ys[i], xs[i], problems[i][0], problems[i][1], K, G, np.arange(N),
                    "problem %d" % i)


def test_repeatable():
    G = 128
    rng = np.random.default_rng(860)
    shapes = [(3584, 1024)] * 24
    problems = [_problem(rng, N, K, G) for N, K in shapes]
    xs = [inputs.activation(870 + i, 1, 1024) for i in range(24)]
    a, _ = _grouped(problems, xs, G)
    b, _ = _grouped(problems, xs, G)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
