"""The oracle's row-partitioned entry points give the same bits for every
thread count: each output row is computed by the single-thread loop, in k
order, whatever the split (including more threads than rows and one thread
per row).  Status bits found in any part are reported."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs


@pytest.mark.parametrize("threads", [2, 3, 7, 16, 64])
def test_quantize_pack_split_invariant(threads):
    N, K, G = 37, 640, 128
    w = inputs.normal_bf16(91, (N, K), 0.02)
    w[5, 3] = 0x7F80   # +Inf in row 5: NONFINITE from one part
    p1, s1, st1 = oracle.quantize_pack(w, G, threads=1)
    pt, stt_s, stt = oracle.quantize_pack(w, G, threads=threads)
    assert st1 == stt == oracle.NONFINITE
    assert np.array_equal(p1, pt) and np.array_equal(s1, stt_s)


@pytest.mark.parametrize("threads", [2, 5, 16, 100])
def test_matmul_split_invariant(threads):
    N, K, G, M = 45, 384, 64, 3
    w = inputs.normal_bf16(92, (N, K), 0.02)
    x = inputs.activation(93, M, K)
    packed, scales, _ = oracle.quantize_pack(w, G, threads=1)
    packed[44, 7] = 250  # an invalid byte in the last row: seen by the last part only
    y1, b1, st1 = oracle.matmul(x, packed, scales, N, K, G, threads=1)
    yt, bt, stt = oracle.matmul(x, packed, scales, N, K, G, threads=threads)
    assert st1 == stt == oracle.INVALID_BYTE
    assert np.array_equal(y1.view(np.uint64), yt.view(np.uint64))
    assert np.array_equal(b1.view(np.uint64), bt.view(np.uint64))


@pytest.mark.parametrize("threads", [3, 16])
def test_matmul2_and_w4a16_split_invariant(threads):
    N, K, G, M = 29, 256, 128, 2
    w = inputs.normal_bf16(94, (N, K), 0.02)
    x = inputs.activation(95, M, K)
    p2, s2, _ = oracle.quantize_pack2(w, G)
    a = oracle.matmul2(x, p2, s2, N, K, G, threads=1)
    b = oracle.matmul2(x, p2, s2, N, K, G, threads=threads)
    assert a[2] == b[2] and np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    pk, sc, bi = inputs.w4a16_problem(96, N, K, G)
    c = oracle.w4a16_matmul(x, pk, sc, bi, N, K, G, threads=1)
    d = oracle.w4a16_matmul(x, pk, sc, bi, N, K, G, threads=threads)
    assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1])
