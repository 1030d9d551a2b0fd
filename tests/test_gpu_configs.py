"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark times, with every output compared against the CPU oracle:
packed bytes and scales bit for bit, matmul outputs within
|y - y_ref| <= 1e-3 * sum_k |x_k w_hat_k| (y_ref in fp64).

Workloads (seeds in ternary_weight_only_amd.inputs):
  - one Qwen-like FFN block and the 72-matrix stack (24 layers of gate and up
    W[3584,1024] and down W[1024,3584]), G = 64 and 128, decode at M = 1;
  - the prefill GEMM on the stack's shapes at M = 512 and 2048, G = 128
    (the grouped launch over all 72 problems, and per-shape batched launches);
  - the 8B-class FFN matrices W[14336,4096] and W[4096,14336], G = 128,
    decode at M = 1, 4 and 16.
"""
import functools

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import (assert_within_bound, dev_bf16, gpu_matmul, host_u16, say)

import torch
import ternary_weight_only_amd as tq

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _stack():
    say("generating the 72 stack matrices")
    return inputs.stack_weights()


@functools.lru_cache(maxsize=2)
def _stack_ref(G):
    """The oracle's packed bytes and scales of every stack matrix."""
    out = []
    for w in _stack():
        p, s, st = oracle.quantize_pack(w, G)
        assert st == 0
        out.append((p, s))
    return out


def _groups():
    """Indices of the stack matrices per shape, in stack order."""
    g = {}
    for i, NK in enumerate(inputs.stack_shapes()):
        g.setdefault(NK, []).append(i)
    return g


def _quantize_stack_batched(G):
    """The benchmark's quantize launch: one tq_quantize_pack_batched call per
    shape (48 and 24 matrices)."""
    ws = [dev_bf16(w) for w in _stack()]
    st = tq.new_status()
    out = [None] * len(ws)
    for (N, K), idx in _groups().items():
        res = tq.quantize_pack_batched([ws[i] for i in idx], G, status=st)
        for i, r in zip(idx, res):
            out[i] = r
    torch.cuda.synchronize()
    return out, int(st.item())


@pytest.mark.parametrize("G", [64, 128])
def test_ffn_block_decode(G):
    """One FFN block (gate, up [3584,1024]; down [1024,3584]) quantized by
    single calls and decoded at M = 1: every byte, scale and output."""
    for p_idx, (name, N, K) in enumerate(inputs.ffn_shapes()):
        w = _stack()[p_idx]
        say("FFN block %s W[%d,%d] G=%d: quantize + gemv M=1" % (name, N, K, G))
        st = tq.new_status()
        packed, scales = tq.quantize_pack(dev_bf16(w), G, status=st)
        p_ref, s_ref = _stack_ref(G)[p_idx]
        assert np.array_equal(packed.cpu().numpy(), p_ref)
        assert np.array_equal(host_u16(scales), s_ref)
        assert int(st.item()) == 0
        x = inputs.stack_decode_activation(p_idx, K)
        y, st2 = gpu_matmul("gemv", x, p_ref, s_ref, N, K, G)
        y_ref, bound, _ = oracle.matmul(x, p_ref, s_ref, N, K, G)
        assert st2 == 0
        assert_within_bound(y, y_ref, bound, "FFN %s G=%d" % (name, G))


@pytest.mark.parametrize("G", [64, 128])
def test_ffn_stack_quantize_every_byte(G):
    """All 72 stack matrices packed by the benchmark's two batched launches:
    every packed byte and every scale bit-exact."""
    say("stack quantize (batched launches) G=%d" % G)
    out, st = _quantize_stack_batched(G)
    assert st == 0
    for i, ((p, s), (p_ref, s_ref)) in enumerate(zip(out, _stack_ref(G))):
        assert np.array_equal(p.cpu().numpy(), p_ref), "matrix %d: packed bytes" % i
        assert np.array_equal(host_u16(s), s_ref), "matrix %d: scales" % i


@pytest.mark.parametrize("G", [64, 128])
def test_ffn_stack_grouped_decode_every_output(G):
    """The benchmark's decode pass: one tq_gemv_grouped call over all 72
    matrices (48 x W[3584,1024] and 24 x W[1024,3584]) on the packed bytes
    the batched quantize launches wrote; every output within the bound."""
    out, st = _quantize_stack_batched(G)
    assert st == 0
    shapes = inputs.stack_shapes()
    xs = [inputs.stack_decode_activation(i, K) for i, (N, K) in enumerate(shapes)]
    say("stack grouped gemv G=%d" % G)
    yst = tq.new_status()
    ys = tq.gemv_grouped([dev_bf16(x) for x in xs], [p for p, _ in out], [s for _, s in out],
                         [N for N, _ in shapes], [K for _, K in shapes], G, status=yst)
    torch.cuda.synchronize()
    assert int(yst.item()) == 0
    for i, ((N, K), (p_ref, s_ref)) in enumerate(zip(shapes, _stack_ref(G))):
        y_ref, bound, _ = oracle.matmul(xs[i], p_ref, s_ref, N, K, G)
        assert_within_bound(ys[i].cpu().numpy(), y_ref, bound, "grouped stack matrix %d G=%d"
                            % (i, G))


@pytest.mark.parametrize("G", [64, 128])
def test_ffn_stack_batched_decode_every_output(G):
    """The stack decoded with two batched calls (48 gate/up matrices with
    K = 1024, 24 down matrices with K = 3584); every output compared."""
    out, st = _quantize_stack_batched(G)
    assert st == 0
    shapes = inputs.stack_shapes()
    for (N, K), idx in _groups().items():
        xs = [inputs.stack_decode_activation(i, K) for i in idx]
        say("batched stack decode K=%d G=%d count=%d" % (K, G, len(idx)))
        yst = tq.new_status()
        ys = tq.gemv_batched([dev_bf16(x) for x in xs], [out[i][0] for i in idx],
                             [out[i][1] for i in idx], N, K, G, status=yst)
        torch.cuda.synchronize()
        assert int(yst.item()) == 0
        for j, i in enumerate(idx):
            p_ref, s_ref = _stack_ref(G)[i]
            y_ref, bound, _ = oracle.matmul(xs[j], p_ref, s_ref, N, K, G)
            assert_within_bound(ys[j].cpu().numpy(), y_ref, bound,
                                "batched stack matrix %d G=%d" % (i, G))
    assert len(shapes) == 72


@pytest.mark.parametrize("M", [512, 2048])
def test_prefill_gemm_single_every_output(M):
    """Single tq_gemm calls on one gate and one down matrix, G = 128: every
    output compared."""
    G = 128
    for p_idx in (0, 2):
        _, N, K = inputs.ffn_shapes()[p_idx]
        x = inputs.prefill_activation(M, K)
        p_ref, s_ref = _stack_ref(G)[p_idx]
        say("prefill gemm (single call) M=%d W[%d,%d]" % (M, N, K))
        y, st = gpu_matmul("gemm", x, p_ref, s_ref, N, K, G)
        assert st == 0
        y_ref, bound, _ = oracle.matmul(x, p_ref, s_ref, N, K, G)
        assert_within_bound(y, y_ref, bound, "gemm M=%d W[%d,%d]" % (M, N, K))


def _stack_gemm(M, G, launch="grouped"):
    """The benchmark's prefill launch: one tq_gemm_grouped call over all 72
    problems (48 of K = 1024 sharing one x, 24 of K = 3584 sharing another),
    on the packed bytes the batched quantize launches wrote; or
    (launch="batched") one tq_gemm_batched call per shape."""
    out, st = _quantize_stack_batched(G)
    assert st == 0
    xs = {K: inputs.prefill_activation(M, K) for K in (1024, 3584)}
    ys = [None] * len(out)
    yst = tq.new_status()
    if launch == "grouped":
        shapes = inputs.stack_shapes()
        say("stack prefill gemm M=%d grouped x %d" % (M, len(shapes)))
        xd = {K: dev_bf16(x) for K, x in xs.items()}
        ys = tq.gemm_grouped([xd[K] for _, K in shapes], [p for p, _ in out], [s for _, s in out],
                             [N for N, _ in shapes], [K for _, K in shapes], G, status=yst)
        torch.cuda.synchronize()
        assert int(yst.item()) == 0
        return xs, ys
    for (N, K), idx in _groups().items():
        say("stack prefill gemm M=%d W[%d,%d] x %d" % (M, N, K, len(idx)))
        xd = dev_bf16(xs[K])
        res = tq.gemm_batched([xd] * len(idx), [out[i][0] for i in idx], [out[i][1] for i in idx],
                              N, K, G, status=yst)
        for i, y in zip(idx, res):
            ys[i] = y
    torch.cuda.synchronize()
    assert int(yst.item()) == 0
    return xs, ys


@pytest.mark.parametrize("launch", ["grouped", "batched"])
def test_prefill_gemm_stack_m512_every_output(launch):
    """M = 512: every output of all 72 problems of the benchmark's grouped
    launch, and of the two batched launches (one per shape)."""
    G, M = 128, 512
    xs, ys = _stack_gemm(M, G, launch)
    for i, (N, K) in enumerate(inputs.stack_shapes()):
        p_ref, s_ref = _stack_ref(G)[i]
        y_ref, bound, _ = oracle.matmul(xs[K], p_ref, s_ref, N, K, G)
        assert_within_bound(ys[i].cpu().numpy(), y_ref, bound, "stack gemm M=512 matrix %d" % i)


@pytest.mark.parametrize("part", range(4))
def test_prefill_gemm_stack_m2048_every_output(part):
    """M = 2048, the same grouped launch over all 72 problems: every output
    of the problems i with i % 4 == part (the oracle's cost split over four
    cases)."""
    G, M = 128, 2048
    xs, ys = _stack_gemm(M, G)
    for i, (N, K) in enumerate(inputs.stack_shapes()):
        if i % 4 != part:
            continue
        p_ref, s_ref = _stack_ref(G)[i]
        y_ref, bound, _ = oracle.matmul(xs[K], p_ref, s_ref, N, K, G)
        assert_within_bound(ys[i].cpu().numpy(), y_ref, bound, "stack gemm M=2048 matrix %d" % i)


@pytest.mark.parametrize("shape", [(14336, 4096), (4096, 14336)])
def test_8b_class_ffn_every_output(shape):
    """8B-class dense FFN matrix at G = 128: every packed byte and scale, and
    every output of the decode at M = 1, 4 and 16."""
    N, K = shape
    G = 128
    w = inputs.dense8b_weight(N, K)
    say("8B-class W[%d,%d]: quantize" % (N, K))
    st = tq.new_status()
    packed, scales = tq.quantize_pack(dev_bf16(w), G, status=st)
    p_ref, s_ref, st_ref = oracle.quantize_pack(w, G)
    assert int(st.item()) == st_ref == 0
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(host_u16(scales), s_ref)
    for M in (1, 4, 16):
        say("8B-class W[%d,%d]: gemv M=%d" % (N, K, M))
        x = inputs.dense8b_activation(M, N, K)
        yst = tq.new_status()
        y = tq.gemv(dev_bf16(x), packed, scales, N, K, G, status=yst)
        torch.cuda.synchronize()
        assert int(yst.item()) == 0
        y_ref, bound, _ = oracle.matmul(x, p_ref, s_ref, N, K, G)
        assert_within_bound(y.cpu().numpy(), y_ref, bound, "8B W[%d,%d] M=%d" % (N, K, M))
