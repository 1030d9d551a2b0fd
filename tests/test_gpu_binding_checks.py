"""The binding rejects, before any launch, every caller-supplied output and
status word the library would write out of bounds or to host memory: wrong
size, wrong dtype, non-contiguous, on the host, or (for status) not int32.
Each case checks that the output's memory is untouched (no kernel ran)."""
import numpy as np
import pytest
import torch

import ternary_weight_only_amd as tq
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import dev_bf16, say

pytestmark = pytest.mark.gpu

N, K, G = 64, 256, 64


def _inputs():
    w = dev_bf16(inputs.normal_bf16(61, (N, K), 0.02))
    x = dev_bf16(inputs.activation(62, 2, K))
    packed, scales = tq.quantize_pack(w, G)
    torch.cuda.synchronize()
    return w, x, packed, scales


def _bad_status():
    return [torch.zeros(1, dtype=torch.int64, device="cuda"),      # wrong dtype
            torch.zeros(1, dtype=torch.int32),                     # host memory
            torch.zeros(0, dtype=torch.int32, device="cuda"),      # empty
            torch.zeros(4, dtype=torch.int32, device="cuda")[::2]]  # not contiguous


def test_bad_status_words_rejected():
    w, x, packed, scales = _inputs()
    say("binding checks: status words")
    for st in _bad_status():
        for call in (lambda: tq.quantize_pack(w, G, status=st),
                     lambda: tq.unpack(packed, N, K, G, status=st),
                     lambda: tq.gemv(x, packed, scales, N, K, G, status=st),
                     lambda: tq.gemm(x, packed, scales, N, K, G, status=st),
                     lambda: tq.dequantize(packed, scales, N, K, G, status=st),
                     lambda: tq.gemv_grouped([x[:1]], [packed], [scales], [N], [K], G, status=st)):
            with pytest.raises(tq.TQError):
                call()


def test_bad_matmul_outputs_rejected():
    w, x, packed, scales = _inputs()
    say("binding checks: matmul outputs")
    sentinel = 3.0   # exact in every dtype used below
    bad = [torch.full((2, N - 1), sentinel, device="cuda"),                   # short
           torch.full((2, N), sentinel, dtype=torch.bfloat16, device="cuda"),  # dtype
           torch.full((2, N), sentinel),                                      # host
           torch.full((N, 4), sentinel, device="cuda").t()]                   # strided
    for y in bad:
        for fn in (tq.gemv, tq.gemm):
            with pytest.raises(tq.TQError):
                fn(x, packed, scales, N, K, G, out=y)
        torch.cuda.synchronize()
        assert bool((y.float() == sentinel).all()), "a rejected output was written"
    with pytest.raises(tq.TQError):
        tq.gemm_batched([x, x], [packed, packed], [scales, scales], N, K, G,
                        outs=[torch.empty(2, N, device="cuda")])            # one output short
    with pytest.raises(tq.TQError):
        tq.gemv_batched([x], [packed], [scales], N, K, G,
                        outs=[torch.empty(2, N + 1, device="cuda")])
    with pytest.raises(tq.TQError):
        tq.gemv_grouped([x[:1]], [packed], [scales], [N], [K], G,
                        outs=[torch.empty(1, N, dtype=torch.float16, device="cuda")])


def test_bad_codec_outputs_rejected():
    w, x, packed, scales = _inputs()
    say("binding checks: quantize / unpack / decode outputs")
    rb = tq.packed_row_bytes(K, G)
    assert rb == (K // G) * 13 and tq.packed_bytes(N, K, G) == N * rb
    with pytest.raises(tq.TQError):
        tq.quantize_pack(w, G, out=(torch.empty(N, rb - 1, dtype=torch.uint8, device="cuda"),
                                    torch.empty(N, K // G, dtype=torch.float16, device="cuda")))
    with pytest.raises(tq.TQError):
        tq.quantize_pack(w, G, out=(torch.empty(N, rb, dtype=torch.uint8, device="cuda"),
                                    torch.empty(N, K // G, dtype=torch.float32, device="cuda")))
    with pytest.raises(tq.TQError):
        tq.unpack(packed, N, K, G, out=torch.empty(N, K - 1, dtype=torch.int8, device="cuda"))
    with pytest.raises(tq.TQError):
        tq.unpack(packed, N, K, G, out=torch.empty(N, K, dtype=torch.uint8, device="cuda"))
    with pytest.raises(tq.TQError):
        tq.dequantize(packed, scales, N, K, G,
                      out=torch.empty(N, K, dtype=torch.float16, device="cuda"))
    with pytest.raises(tq.TQError):
        tq.fake_quantize(w, G, out=torch.empty(N, K // 2, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(tq.TQError):
        tq.fake_quantize(w, G, scales_out=torch.empty(N, K // G - 1, dtype=torch.float16,
                                                      device="cuda"))
    with pytest.raises(tq.TQError):
        tq.dequantize_batched([packed], [scales], N, K, G,
                              outs=[torch.empty(N, K, dtype=torch.bfloat16)])


def test_good_outputs_accepted():
    """Outputs of the right size given as other shapes or as int16 bit
    patterns are accepted and written."""
    w, x, packed, scales = _inputs()
    say("binding checks: valid caller outputs")
    y = torch.empty(2 * N, device="cuda")
    tq.gemm(x, packed, scales, N, K, G, out=y)
    y2 = tq.gemm(x, packed, scales, N, K, G)
    torch.cuda.synchronize()
    assert torch.equal(y.view(2, N), y2)
    codes = torch.empty(N * K, dtype=torch.int8, device="cuda")
    tq.unpack(packed, N, K, G, out=codes)
    assert torch.equal(codes.view(N, K), tq.unpack(packed, N, K, G))
