"""GPU parity of the W4A16 matmul for any number of rows (tq_w4a16_gemm) and
of the W4A16 GEMV on rows longer than 4096, against the CPU oracle's fp64
sum in the page's order (tiny-llm "Week 2 Day 3: Quantize the Model":
"Group-Wise Affine Quantization", "Packed Storage Layout", "Mathematical
Formulation", "Computation Flow", "GPU Dispatch").

Bar, as for the W4A16 GEMV: |y - y_ref| <= 1e-3 * B * (1 + 2^-8) + 2^-8 |y_ref|
with B = sum_k |x| (|q s| + |b|); every output compared unless noted."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import dev_bf16, host_u16, say
from tests.test_gpu_w4a16 import bf16_val, dev_u32
from tests.test_oracle_w4a16 import random_problem

pytestmark = pytest.mark.gpu


def _check(y_bits, y_ref, bound, what):
    y = bf16_val(y_bits)
    tol = 1e-3 * bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y_ref)
    bad = ~(np.abs(y - y_ref) <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d outside the bar; first at %s: gpu=%r ref=%r tol=%r"
                             % (what, int(bad.sum()), bad.size, i, y[i], y_ref[i], tol[i]))


def _gemm(x, packed, s, b, N, K, G):
    import torch
    import ternary_weight_only_amd as tq
    y = tq.w4a16_gemm(dev_bf16(x), dev_u32(packed), dev_bf16(s), dev_bf16(b), N, K, G)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("M,N,K,G", [(1, 300, 640, 64), (2, 3584, 1024, 128), (3, 1024, 3584, 128),
                                     (8, 129, 8192, 128), (16, 1000, 4096, 64),
                                     (17, 250, 1024, 128), (33, 77, 640, 64),
                                     (100, 513, 1088, 64), (512, 3584, 1024, 128),
                                     (512, 1024, 3584, 128)])
def test_w4a16_gemm_parity(M, N, K, G):
    """Few-row (16-row tiles) and many-row (64-row tiles) launches, ragged M
    and N, K past 4096, both G."""
    packed, s, b = random_problem(500 + N + M, N, K, G)
    x = inputs.activation(501 + K + M, M, K)
    say("w4a16 gemm M=%d W[%d,%d] G=%d" % (M, N, K, G))
    y = _gemm(x, packed, s, b, N, K, G)
    y_ref, bound = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
    _check(y, y_ref, bound, "M=%d W[%d,%d] G=%d" % (M, N, K, G))


def test_w4a16_gemm_prefill_m2048_every_output():
    """M = 2048 on the FFN's gate shape: every output."""
    M, N, K, G = 2048, 3584, 1024, 128
    packed, s, b = inputs.w4a16_problem(520, N, K, G)
    x = inputs.activation(521, M, K)
    say("w4a16 gemm M=2048")
    y = _gemm(x, packed, s, b, N, K, G)
    y_ref, bound = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
    _check(y, y_ref, bound, "M=2048")


@pytest.mark.parametrize("N,K", [(4096, 14336), (37, 8192)])
def test_w4a16_gemv_long_rows(N, K):
    """tq_w4a16_gemv on rows past 4096 (the 8B-class down projection): the
    matrix-core kernel at M = 1, equal bit for bit to tq_w4a16_gemm."""
    import torch
    import ternary_weight_only_amd as tq
    G = 128
    packed, s, b = inputs.w4a16_problem(530 + N, N, K, G)
    x = inputs.activation(531, 1, K)
    say("w4a16 gemv long rows W[%d,%d]" % (N, K))
    args = (dev_bf16(x), dev_u32(packed), dev_bf16(s), dev_bf16(b), N, K, G)
    y1 = tq.w4a16_gemv(*args)
    y2 = tq.w4a16_gemm(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y_ref, bound = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
    _check(host_u16(y1), y_ref, bound, "gemv W[%d,%d]" % (N, K))


def test_w4a16_grouped_and_batched_with_long_rows():
    """Grouped calls mixing table-kernel shapes with K = 8192 rows, and a
    batched call at K = 6144: each result bit-identical to its single call."""
    import torch
    import ternary_weight_only_amd as tq
    G = 64
    shapes = [(200, 1024), (64, 8192), (300, 4096), (16, 8192)]
    probs = [random_problem(540 + i, N, K, G) for i, (N, K) in enumerate(shapes)]
    xs = [dev_bf16(inputs.activation(550 + i, 1, K)) for i, (N, K) in enumerate(shapes)]
    dv = [(dev_u32(p), dev_bf16(s), dev_bf16(b)) for p, s, b in probs]
    say("w4a16 grouped with long rows")
    ys = tq.w4a16_gemv_grouped(xs, [d[0] for d in dv], [d[1] for d in dv], [d[2] for d in dv],
                               [N for N, _ in shapes], [K for _, K in shapes], G)
    for i, (N, K) in enumerate(shapes):
        y1 = tq.w4a16_gemv(xs[i], dv[i][0], dv[i][1], dv[i][2], N, K, G)
        torch.cuda.synchronize()
        assert torch.equal(ys[i], y1), i
    N, K = 96, 6144
    bp = [random_problem(560 + i, N, K, G) for i in range(3)]
    bx = [dev_bf16(inputs.activation(570 + i, 1, K)) for i in range(3)]
    bd = [(dev_u32(p), dev_bf16(s), dev_bf16(b)) for p, s, b in bp]
    yb = tq.w4a16_gemv_batched(bx, [d[0] for d in bd], [d[1] for d in bd], [d[2] for d in bd],
                               N, K, G)
    for i in range(3):
        y1 = tq.w4a16_gemv(bx[i], bd[i][0], bd[i][1], bd[i][2], N, K, G)
        torch.cuda.synchronize()
        assert torch.equal(yb[i], y1), i
        xh = host_u16(bx[i])
        y_ref, bound = oracle.w4a16_matmul(xh, bp[i][0], bp[i][1], bp[i][2], N, K, G)
        _check(host_u16(yb[i])[0], y_ref[0], bound[0], "batched %d" % i)


def test_w4a16_gemm_nonfinite_parameter_stays_in_its_row():
    """A NaN scale in row 5 and an Inf bias in row 9: those columns of y are
    non-finite, every other output meets the bar."""
    M, N, K, G = 20, 64, 512, 128
    packed, s, b = random_problem(580, N, K, G)
    s = s.copy()
    b = b.copy()
    s[5, 1] = 0x7FC0
    b[9, 2] = 0x7F80
    x = inputs.activation(581, M, K)
    say("w4a16 gemm non-finite parameters")
    y = bf16_val(_gemm(x, packed, s, b, N, K, G))
    assert not np.isfinite(y[:, 5]).any() and not np.isfinite(y[:, 9]).any()
    keep = [n for n in range(N) if n not in (5, 9)]
    ok = np.ones(N, bool)
    ok[[5, 9]] = False
    s2, b2 = s.copy(), b.copy()
    s2[5, 1] = 0
    b2[9, 2] = 0
    y_ref, bound = oracle.w4a16_matmul(x, packed, s2, b2, N, K, G)
    tol = 1e-3 * bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y_ref)
    assert (np.abs(y[:, keep] - y_ref[:, keep]) <= tol[:, keep]).all()


@pytest.mark.parametrize("M,N,K,G,count", [(5, 300, 640, 64, 3), (40, 1024, 3584, 128, 2),
                                           (512, 1024, 3584, 128, 3), (1, 200, 8192, 128, 2),
                                           (1, 256, 1024, 128, 3)])
def test_w4a16_gemm_batched(M, N, K, G, count):
    """Batched launches (the problems on the grid's z axis, or the table GEMV
    at M = 1 with K <= 4096): every output bit-identical to single calls and
    within the bar."""
    import torch
    import ternary_weight_only_amd as tq
    probs = [random_problem(600 + 7 * i + M, N, K, G) for i in range(count)]
    xs = [inputs.activation(650 + 7 * i + K, M, K) for i in range(count)]
    say("w4a16 gemm batched M=%d W[%d,%d] G=%d x%d" % (M, N, K, G, count))
    ys = tq.w4a16_gemm_batched([dev_bf16(x) for x in xs], [dev_u32(p) for p, _, _ in probs],
                               [dev_bf16(s) for _, s, _ in probs],
                               [dev_bf16(b) for _, _, b in probs], N, K, G)
    torch.cuda.synchronize()
    for i, ((packed, s, b), x, y) in enumerate(zip(probs, xs, ys)):
        yb = host_u16(y)
        assert np.array_equal(yb, _gemm(x, packed, s, b, N, K, G)), "problem %d" % i
        y_ref, bound = oracle.w4a16_matmul(x, packed, s, b, N, K, G)
        _check(yb, y_ref, bound, "batched problem %d" % i)
