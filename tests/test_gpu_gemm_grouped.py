"""GPU parity of the grouped prefill matmul (tq_gemm_grouped): problems of
different N and K that share M, in one persistent launch where the 256 x 128
tile kernel takes every shape, else one batched launch per shape.  Every
output is compared with the CPU oracle's fp64 result within
|y - y_ref| <= 1e-3 * sum_k |x_k w_hat_k| (tiny-llm "Week 2 Day 3: Quantize
the Model", "Mathematical Formulation").

Cases: five shapes in one call (more than one launch's four), ragged M and N,
K from 256 to 1536; more than 128 problems (two launches); the fallback
(G = 64, and M below one 256-row tile); an invalid packed byte in one
problem; an empty call."""
import functools

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import assert_within_bound, dev_bf16, dev_f16bits, dev_u8, say

import torch
import ternary_weight_only_amd as tq

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=32)
def _packed(seed, N, K, G):
    w = inputs.normal_bf16(seed, (N, K), inputs.W_SIGMA)
    p, s, st = oracle.quantize_pack(w, G)
    assert st == 0
    return p, s


def _tiles(M, Ns):
    return sum(((M + 255) // 256) * ((N + 127) // 128) for N in Ns)


def _run(M, shapes, G, seed, bad=None):
    """shapes: list of (N, K) per problem; every problem has its own x.
    bad: index of a problem whose first packed byte is made invalid."""
    xs, ps, ss = [], [], []
    for i, (N, K) in enumerate(shapes):
        p, s = _packed(seed + 7 * i, N, K, G)
        if bad == i:
            p = p.copy()
            p.reshape(-1)[0] = 255
        xs.append(inputs.activation(seed + 1000 + i, M, K))
        ps.append(p)
        ss.append(s)
    st = tq.new_status()
    ys = tq.gemm_grouped([dev_bf16(x) for x in xs], [dev_u8(p) for p in ps],
                         [dev_f16bits(s) for s in ss], [N for N, _ in shapes],
                         [K for _, K in shapes], G, status=st)
    torch.cuda.synchronize()
    return xs, ps, ss, [y.cpu().numpy() for y in ys], int(st.item())


def _check_all(M, shapes, G, xs, ps, ss, ys, what, skip=()):
    for i, (N, K) in enumerate(shapes):
        if i in skip:
            continue
        assert ys[i].shape == (M, N)
        y_ref, bound, _ = oracle.matmul(xs[i], ps[i], ss[i], N, K, G)
        assert_within_bound(ys[i], y_ref, bound, "%s problem %d W[%d,%d]" % (what, i, N, K))


@pytest.mark.parametrize("M", [520, 777])
def test_grouped_five_shapes_every_output(M):
    """Ten problems of five shapes, interleaved in the call: two launches
    (four shapes, then one), longest K first within each."""
    G = 128
    A, B, C, D, E = (2048, 1024), (512, 1536), (1000, 640), (130, 1152), (77, 256)
    shapes = [A, C, B, A, E, D, C, A, B, E]
    assert _tiles(M, [N for N, _ in shapes]) >= 192  # the persistent grouped launch
    say("gemm_grouped M=%d five shapes" % M)
    xs, ps, ss, ys, st = _run(M, shapes, G, 3100)
    assert st == 0
    _check_all(M, shapes, G, xs, ps, ss, ys, "grouped M=%d" % M)


def test_grouped_more_than_128_problems():
    """130 problems of two shapes at M = 256: the problems fill one launch of
    128 and spill into a second."""
    G, M = 128, 256
    shapes = [(256, 256) if i % 3 else (384, 128) for i in range(130)]
    assert _tiles(M, [N for N, _ in shapes]) >= 192
    say("gemm_grouped M=256 130 problems")
    xs, ps, ss, ys, st = _run(M, shapes, G, 3200)
    assert st == 0
    _check_all(M, shapes, G, xs, ps, ss, ys, "grouped x130")


@pytest.mark.parametrize("M,G", [(512, 64), (100, 128), (1, 128)])
def test_grouped_fallback_every_output(M, G):
    """Shapes the 256 x 128 kernel does not take run one batched call per
    shape; the result is the same computation."""
    shapes = [(1000, 640), (384, 1024), (1000, 640), (200, 384)]
    say("gemm_grouped fallback M=%d G=%d" % (M, G))
    xs, ps, ss, ys, st = _run(M, shapes, G, 3300)
    assert st == 0
    _check_all(M, shapes, G, xs, ps, ss, ys, "grouped fallback M=%d G=%d" % (M, G))


def test_grouped_invalid_byte_flags_status():
    """A byte of 255 in one problem sets INVALID_BYTE; the other problems'
    outputs stay exact to the bound."""
    G, M = 128, 512
    shapes = [(3584, 1024), (1024, 2048), (3584, 1024), (3584, 1024), (3584, 1024)]
    assert _tiles(M, [N for N, _ in shapes]) >= 192
    say("gemm_grouped invalid byte")
    xs, ps, ss, ys, st = _run(M, shapes, G, 3400, bad=1)
    assert st & tq.DEV_INVALID_BYTE
    _check_all(M, shapes, G, xs, ps, ss, ys, "grouped invalid byte", skip=(1,))


def test_grouped_empty():
    assert tq.gemm_grouped([], [], [], [], [], 128) == []
