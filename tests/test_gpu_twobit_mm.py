"""GPU parity of the 2-bit format's matrix-core matmul (tq_gemm2,
tq_gemm2_batched; any M, any K) and of the 2-bit GEMV on rows longer than
4096 (which runs it), against the CPU oracle's fp64 result.

Format: fields c + 1 in two bits, four a byte, first weight lowest (Avenue
README, size note on 2-bit packing; "Autoregressive Language Model on the
6502 Processor"); a field of 3 counts as code 0 and sets INVALID_BYTE.
Bar: |y - y_ref| <= 1e-3 * sum_k |x_k w_hat_k| per element (tiny-llm "Week 2
Day 3: Quantize the Model", "Mathematical Formulation"); every output
compared."""
import functools

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import assert_within_bound, dev_bf16, dev_f16bits, dev_u8, say

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=8)
def _packed(seed, N, K, G):
    w = inputs.normal_bf16(seed, (N, K), inputs.W_SIGMA)
    p, s, st = oracle.quantize_pack2(w, G)
    assert st == 0
    return p, s


def _gemm2(x, p, s, N, K, G):
    import torch
    import ternary_weight_only_amd as tq
    st = tq.new_status()
    y = tq.gemm2(dev_bf16(x), dev_u8(p), dev_f16bits(s), N, K, G, status=st)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(st.item())


@pytest.mark.parametrize("M,N,K,G", [(1, 300, 8192, 128), (2, 3584, 1024, 128),
                                     (5, 129, 640, 64), (16, 1000, 4096, 64),
                                     (17, 250, 1024, 128), (33, 77, 640, 64),
                                     (100, 513, 1088, 64), (512, 1024, 3584, 128)])
def test_gemm2_parity(M, N, K, G):
    """Few-row (16-row tiles) and many-row (32- and 64-row tiles) launches,
    ragged M and N, rows past 4096, both G."""
    p, s = _packed(700 + N, N, K, G)
    x = inputs.activation(701 + M + K, M, K)
    say("gemm2 M=%d W[%d,%d] G=%d" % (M, N, K, G))
    y, st = _gemm2(x, p, s, N, K, G)
    assert st == 0
    y_ref, bound, _ = oracle.matmul2(x, p, s, N, K, G)
    assert_within_bound(y, y_ref, bound, "gemm2 M=%d W[%d,%d] G=%d" % (M, N, K, G))


@pytest.mark.parametrize("shape", [(14336, 4096), (4096, 14336)])
def test_gemm2_8b_class_every_output(shape):
    """The 8B-class FFN matrices in the 2-bit format at M = 1, 4 and 16 (M = 1
    through tq_gemv2: the table kernel for K = 4096, the matrix-core kernel for
    K = 14336)."""
    import torch
    import ternary_weight_only_amd as tq
    N, K = shape
    G = 128
    w = inputs.dense8b_weight(N, K)
    p, s, st = oracle.quantize_pack2(w, G)
    assert st == 0
    for M in (1, 4, 16):
        x = inputs.dense8b_activation(M, N, K)
        say("2-bit 8B-class W[%d,%d] M=%d" % (N, K, M))
        if M == 1:
            yst = tq.new_status()
            yd = tq.gemv2(dev_bf16(x), dev_u8(p), dev_f16bits(s), N, K, G, status=yst)
            torch.cuda.synchronize()
            y, st2 = yd.cpu().numpy(), int(yst.item())
        else:
            y, st2 = _gemm2(x, p, s, N, K, G)
        assert st2 == 0
        y_ref, bound, _ = oracle.matmul2(x, p, s, N, K, G, threads=16)
        assert_within_bound(y, y_ref, bound, "2-bit W[%d,%d] M=%d" % (N, K, M))


@pytest.mark.parametrize("M,K", [(3, 1024), (1, 8192)])
def test_gemm2_invalid_field(M, K):
    """A byte with a field of 3 sets INVALID_BYTE; the field counts as code 0,
    as in the oracle, so every output still meets the bar."""
    N, G = 200, 128
    p, s = _packed(710 + K, N, K, G)
    p = p.copy()
    p[57, 5] = 0xFF          # four fields of 3
    p[N - 1, K // 4 - 1] |= 0x30  # field 2 of the last byte
    x = inputs.activation(711 + K, M, K)
    y, st = _gemm2(x, p, s, N, K, G)
    assert st == 4
    y_ref, bound, st_ref = oracle.matmul2(x, p, s, N, K, G)
    assert st_ref == 4
    assert_within_bound(y, y_ref, bound, "gemm2 with invalid fields")


@pytest.mark.parametrize("bad", [False, True])
def test_gemm2_persistent_launch_every_output(bad):
    """Launches with enough 256 x 128 tiles (12 problems W[1000,1024] at
    M = 260: 192 tiles, ragged in M and N) run on the persistent matrix-core
    kernel shared with the base-3 format; every output of every problem is
    checked, and with `bad` one problem holds fields of 3 (INVALID_BYTE, the
    field counting as code 0)."""
    import torch
    import ternary_weight_only_amd as tq
    M, N, K, G, count = 260, 1000, 1024, 128, 12
    probs = [_packed(760 + i, N, K, G) for i in range(count)]
    if bad:
        p0 = probs[5][0].copy()
        p0[3, 7] = 0xFF
        p0[N - 1, K // 4 - 1] |= 0xC0
        probs[5] = (p0, probs[5][1])
    xs = [inputs.activation(770 + i, M, K) for i in range(count)]
    say("gemm2 persistent M=%d W[%d,%d] x%d bad=%d" % (M, N, K, count, bad))
    st = tq.new_status()
    ys = tq.gemm2_batched([dev_bf16(x) for x in xs], [dev_u8(p) for p, _ in probs],
                          [dev_f16bits(s) for _, s in probs], N, K, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == (4 if bad else 0)
    for i, ((p, s), x, y) in enumerate(zip(probs, xs, ys)):
        y_ref, bound, st_ref = oracle.matmul2(x, p, s, N, K, G, threads=16)
        assert st_ref == (4 if bad and i == 5 else 0)
        assert_within_bound(y.cpu().numpy(), y_ref, bound, "gemm2 persistent problem %d" % i)


@pytest.mark.parametrize("M,N,K,G,count", [(4, 300, 640, 64, 3), (64, 1024, 3584, 128, 2),
                                           (1, 200, 8192, 128, 3), (1, 256, 1024, 128, 2)])
def test_gemm2_batched_equals_single(M, N, K, G, count):
    """Batched launches: every output bit-identical to single calls."""
    import torch
    import ternary_weight_only_amd as tq
    probs = [_packed(720 + i, N, K, G) for i in range(count)]
    xs = [inputs.activation(730 + i + M, M, K) for i in range(count)]
    say("gemm2 batched M=%d W[%d,%d] x%d" % (M, N, K, count))
    st = tq.new_status()
    ys = tq.gemm2_batched([dev_bf16(x) for x in xs], [dev_u8(p) for p, _ in probs],
                          [dev_f16bits(s) for _, s in probs], N, K, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, ((p, s), x, y) in enumerate(zip(probs, xs, ys)):
        y1, _ = _gemm2(x, p, s, N, K, G)
        assert np.array_equal(y.cpu().numpy(), y1), "problem %d" % i


def test_gemv2_grouped_mixed_row_lengths():
    """One grouped 2-bit GEMV call over rows the table kernel takes (K =
    1024) and rows it does not (K = 8192): every output within the bar."""
    import torch
    import ternary_weight_only_amd as tq
    G = 128
    shapes = [(300, 1024), (200, 8192), (100, 1024), (64, 6144)]
    probs = [_packed(740 + i, N, K, G) for i, (N, K) in enumerate(shapes)]
    xs = [inputs.activation(750 + i, 1, K) for i, (N, K) in enumerate(shapes)]
    st = tq.new_status()
    ys = tq.gemv2_grouped([dev_bf16(x) for x in xs], [dev_u8(p) for p, _ in probs],
                          [dev_f16bits(s) for _, s in probs], [N for N, _ in shapes],
                          [K for _, K in shapes], G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, ((N, K), (p, s), x, y) in enumerate(zip(shapes, probs, xs, ys)):
        y_ref, bound, _ = oracle.matmul2(x, p, s, N, K, G)
        assert_within_bound(y.cpu().numpy(), y_ref, bound, "grouped problem %d" % i)
