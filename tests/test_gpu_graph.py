"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
quantize + pack, unpack, the grouped prefill matmul and the grouped decode
GEMV are recorded once, then replayed three times with new weights and
activations written eagerly (and the device synchronised) between replays.
Every replay's outputs equal an eager run on the same inputs bit for bit (the
kernels are deterministic), and the first replay's are checked against the
oracle: packing bit-exact, matmuls within |y - y_ref| <= 1e-3 * sum_k |x_k w_hat_k|
(tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation").
The library allocates nothing and issues no memset, so its calls can be
captured; the status word is cleared eagerly before each replay."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import assert_within_bound, dev_bf16, dev_f16bits, dev_u8, say

import torch
import ternary_weight_only_amd as tq

pytestmark = pytest.mark.gpu

G = 128
SHAPES = [(512, 1024), (384, 1280), (512, 1024)]  # (N, K) of the matmuls
QN, QK = 384, 1024                                # the quantized / unpacked matrix
MP = 300                                          # prefill rows


def _host_inputs(seed):
    w = inputs.normal_bf16(seed, (QN, QK), inputs.W_SIGMA)
    packs = [oracle.quantize_pack(inputs.normal_bf16(seed + 1 + i, (N, K), inputs.W_SIGMA), G)
             for i, (N, K) in enumerate(SHAPES)]
    x1 = [inputs.activation(seed + 10 + i, 1, K) for i, (_, K) in enumerate(SHAPES)]
    xm = [inputs.activation(seed + 20 + i, MP, K) for i, (_, K) in enumerate(SHAPES)]
    return w, packs, x1, xm


def test_graph_replays_equal_eager_runs():
    dev_w = torch.empty((QN, QK), dtype=torch.bfloat16, device="cuda")
    dev_p = [torch.empty((N, tq.packed_row_bytes(K, G)), dtype=torch.uint8, device="cuda")
             for N, K in SHAPES]
    dev_s = [torch.empty((N, K // G), dtype=torch.float16, device="cuda") for N, K in SHAPES]
    dev_x1 = [torch.empty((1, K), dtype=torch.bfloat16, device="cuda") for _, K in SHAPES]
    dev_xm = [torch.empty((MP, K), dtype=torch.bfloat16, device="cuda") for _, K in SHAPES]
    Ns, Ks = [N for N, _ in SHAPES], [K for _, K in SHAPES]
    st = tq.new_status()

    def outputs():
        return ((torch.empty((QN, tq.packed_row_bytes(QK, G)), dtype=torch.uint8, device="cuda"),
                 torch.empty((QN, QK // G), dtype=torch.float16, device="cuda")),
                torch.empty((QN, QK), dtype=torch.int8, device="cuda"),
                [torch.empty((MP, N), dtype=torch.float32, device="cuda") for N in Ns],
                [torch.empty((1, N), dtype=torch.float32, device="cuda") for N in Ns])

    def run(out):
        packed_q, codes, ym, y1 = out
        tq.quantize_pack(dev_w, G, status=st, out=packed_q)
        tq.unpack(packed_q[0], QN, QK, G, status=st, out=codes)
        tq.gemm_grouped(dev_xm, dev_p, dev_s, Ns, Ks, G, status=st, outs=ym)
        tq.gemv_grouped(dev_x1, dev_p, dev_s, Ns, Ks, G, status=st, outs=y1)

    def load(seed):
        w, packs, x1, xm = _host_inputs(seed)
        dev_w.copy_(dev_bf16(w))
        for i, (p, s, _) in enumerate(packs):
            dev_p[i].copy_(dev_u8(p))
            dev_s[i].copy_(dev_f16bits(s))
            dev_x1[i].copy_(dev_bf16(x1[i]))
            dev_xm[i].copy_(dev_bf16(xm[i]))
        return w, packs, x1, xm

    def poison(out):
        packed_q, codes, ym, y1 = out
        packed_q[0].fill_(0xEE)
        packed_q[1].fill_(float("nan"))
        codes.fill_(7)
        for y in ym + y1:
            y.fill_(float("nan"))

    captured = outputs()
    load(4000)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(captured)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(captured)
    torch.cuda.synchronize()

    eager = outputs()
    for rep in range(3):
        say("graph replay %d" % rep)
        host = load(4100 + 17 * rep)
        poison(captured)
        st.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        poison(eager)
        run(eager)
        torch.cuda.synchronize()
        (cp, cs), cc, cym, cy1 = captured
        (ep, es), ec, eym, ey1 = eager
        assert torch.equal(cp, ep) and torch.equal(cs.view(torch.int16), es.view(torch.int16))
        assert torch.equal(cc, ec)
        for a, b in zip(cym + cy1, eym + ey1):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        if rep == 0:
            w, packs, x1, xm = host
            p_ref, s_ref, _ = oracle.quantize_pack(w, G)
            assert np.array_equal(cp.cpu().numpy(), p_ref)
            assert np.array_equal(cs.cpu().view(torch.int16).numpy().view(np.uint16), s_ref)
            assert np.array_equal(cc.cpu().numpy(), oracle.unpack(p_ref, QN, QK, G)[0])
            for i, (N, K) in enumerate(SHAPES):
                p, s, _ = packs[i]
                y_ref, bound, _ = oracle.matmul(x1[i], p, s, N, K, G)
                assert_within_bound(cy1[i].cpu().numpy(), y_ref, bound, "graph gemv %d" % i)
                y_ref, bound, _ = oracle.matmul(xm[i], p, s, N, K, G)
                assert_within_bound(cym[i].cpu().numpy(), y_ref, bound, "graph gemm %d" % i)
