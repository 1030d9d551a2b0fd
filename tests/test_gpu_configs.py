"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (the library picks its launch shape from the call alone).

Outputs too large for the oracle to recompute whole are checked on sampled
rows, which the oracle computes one by one from the same inputs.
"""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import (assert_within_bound, dev_bf16, dev_f16bits, dev_u8, gpu_matmul,
                               host_u16, say)

import torch
import ternary_weight_only_amd as tq

pytestmark = pytest.mark.gpu


def _sample_rows(N, k, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(k, N), replace=False).tolist()) | {0, N - 1}
    return np.array(sorted(rows))


def _quantize_dev(w_bits, G):
    st = tq.new_status()
    packed, scales = tq.quantize_pack(dev_bf16(w_bits), G, status=st)
    return packed, scales, st


def _check_rows_exact(w_bits, packed_d, scales_d, st_d, G, rows, what):
    N, K = w_bits.shape
    p_ref, s_ref, st_ref = oracle.quantize_pack(w_bits[rows], G)
    p = packed_d[torch.from_numpy(rows).cuda()].cpu().numpy()
    s = host_u16(scales_d[torch.from_numpy(rows).cuda()])
    assert np.array_equal(p, p_ref), what + ": packed"
    assert np.array_equal(s, s_ref), what + ": scales"
    assert int(st_d.item()) == 0 and st_ref == 0


def _check_gemv_rows(kind, x_bits, packed_d, scales_d, w_rows_packed, w_rows_scales, N, K, G, rows,
                     what):
    st = tq.new_status()
    fn = tq.gemv if kind == "gemv" else tq.gemm
    y = fn(dev_bf16(x_bits), packed_d, scales_d, N, K, G, status=st).cpu().numpy()
    assert int(st.item()) == 0
    y_ref, bound, _ = oracle.matmul(x_bits, w_rows_packed, w_rows_scales, len(rows), K, G)
    assert_within_bound(y[:, rows], y_ref, bound, what)
    assert np.isfinite(y).all()


@pytest.mark.parametrize("G", [64, 128])
def test_ffn_block_decode(G):
    """One Qwen-like FFN block (gate, up [3584,1024]; down [1024,3584]), M=1:
    every output checked."""
    for p_idx, (name, N, K) in enumerate(inputs.ffn_shapes()):
        w = inputs.ffn_weight(0, p_idx)
        say("FFN block %s W[%d,%d] G=%d: quantize + gemv M=1" % (name, N, K, G))
        packed, scales, st = _quantize_dev(w, G)
        p_ref, s_ref, st_ref = oracle.quantize_pack(w, G)
        assert np.array_equal(packed.cpu().numpy(), p_ref)
        assert np.array_equal(host_u16(scales), s_ref)
        assert int(st.item()) == st_ref == 0
        x = inputs.activation(20 + p_idx, 1, K)
        y, st2 = gpu_matmul("gemv", x, p_ref, s_ref, N, K, G)
        y_ref, bound, _ = oracle.matmul(x, p_ref, s_ref, N, K, G)
        assert st2 == 0
        assert_within_bound(y, y_ref, bound, "FFN %s G=%d" % (name, G))


def test_ffn_stack_72_matrices():
    """24 layers x {gate, up, down}: quantize + pack all 72, GEMV through all
    72 at M=1, for G=64 and G=128; sampled rows checked per matrix."""
    for layer in range(24):
        for p_idx, (name, N, K) in enumerate(inputs.ffn_shapes()):
            w = inputs.ffn_weight(layer, p_idx)
            x = inputs.activation(5000 + 3 * layer + p_idx, 1, K)
            rows = _sample_rows(N, 48, 1000 + 3 * layer + p_idx)
            for G in (64, 128):
                what = "stack layer %d %s G=%d" % (layer, name, G)
                if layer % 8 == 0:
                    say(what)
                packed, scales, st = _quantize_dev(w, G)
                _check_rows_exact(w, packed, scales, st, G, rows, what)
                p_ref, s_ref, _ = oracle.quantize_pack(w[rows], G)
                _check_gemv_rows("gemv", x, packed, scales, p_ref, s_ref, N, K, G, rows, what)


@pytest.mark.parametrize("M", [512, 2048])
def test_prefill_gemm_ffn(M):
    """Prefill GEMM on the FFN shapes, G=128; sampled activation rows x all N."""
    G = 128
    for p_idx, (name, N, K) in enumerate(inputs.ffn_shapes()):
        w = inputs.ffn_weight(0, p_idx)
        x = inputs.activation(30 + p_idx + (3 if M == 2048 else 0), M, K)
        say("prefill gemm M=%d %s W[%d,%d]" % (M, name, N, K))
        packed, scales, st = _quantize_dev(w, G)
        yst = tq.new_status()
        y = tq.gemm(dev_bf16(x), packed, scales, N, K, G, status=yst).cpu().numpy()
        assert int(yst.item()) == 0 and np.isfinite(y).all()
        mrows = _sample_rows(M, 24, 77 + M)
        p_ref, s_ref, _ = oracle.quantize_pack(w, G)
        y_ref, bound, _ = oracle.matmul(x[mrows], p_ref, s_ref, N, K, G)
        assert_within_bound(y[mrows], y_ref, bound, "gemm M=%d %s" % (M, name))


@pytest.mark.parametrize("shape", [(14336, 4096), (4096, 14336)])
def test_8b_class_ffn_batched_gemv(shape):
    """8B-class dense FFN matrices at G=128; batched GEMV at M = 1, 4, 16."""
    N, K = shape
    G = 128
    w = inputs.normal_bf16(40 if N > K else 41, (N, K), 0.02)
    say("8B-class W[%d,%d]: quantize" % (N, K))
    packed, scales, st = _quantize_dev(w, G)
    rows = _sample_rows(N, 96, N)
    _check_rows_exact(w, packed, scales, st, G, rows, "8B W[%d,%d]" % (N, K))
    p_ref, s_ref, _ = oracle.quantize_pack(w[rows], G)
    for i, M in enumerate((1, 4, 16)):
        say("8B-class W[%d,%d]: gemv M=%d" % (N, K, M))
        x = inputs.activation((50 if N > K else 53) + i, M, K)
        _check_gemv_rows("gemv", x, packed, scales, p_ref, s_ref, N, K, G, rows,
                         "8B W[%d,%d] M=%d" % (N, K, M))


@pytest.mark.parametrize("G", [64, 128])
def test_ffn_stack_batched_decode(G):
    """The 72-matrix stack decoded with two batched calls (48 gate/up matrices
    with K=1024, 24 down matrices with K=3584); sampled rows of every matrix
    checked against the oracle."""
    shapes = inputs.ffn_shapes()
    for group in ((0, 1), (2,)):
        _, N, K = shapes[group[0]]
        mats = [(l, p) for l in range(24) for p in group]
        ws = [inputs.ffn_weight(l, p) for l, p in mats]
        xs = [inputs.activation(5000 + 3 * l + p, 1, K) for l, p in mats]
        say("batched stack decode K=%d G=%d count=%d" % (K, G, len(mats)))
        qs = [_quantize_dev(w, G) for w in ws]
        st = tq.new_status()
        ys = tq.gemv_batched([dev_bf16(x) for x in xs], [q[0] for q in qs], [q[1] for q in qs],
                             N, K, G, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        for i, (l, p) in enumerate(mats):
            rows = _sample_rows(N, 24, 7000 + i)
            p_ref, s_ref, _ = oracle.quantize_pack(ws[i][rows], G)
            y_ref, bound, _ = oracle.matmul(xs[i], p_ref, s_ref, len(rows), K, G)
            assert_within_bound(ys[i].cpu().numpy()[:, rows], y_ref, bound,
                                "batched stack layer %d proj %d" % (l, p))
