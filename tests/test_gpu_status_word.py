"""The base-3 decode GEMVs set TQ_DEV_INVALID_BYTE only for a packed byte
>= 243 (include/tq.h), never for non-finite arithmetic: an Inf activation
(Inf * code 0 is NaN) or finite products whose fp32 sums overflow to +Inf
and -Inf and cancel to NaN give NaN outputs and a clear status, at M = 1
(16-lane rows summed in a wave, and 128-lane rows summed across waves) and
at M = 4 (matrix-core kernel).  An invalid byte is still flagged when other
rows are NaN for those reasons."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_only_amd as tq
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import dev_bf16, dev_f16bits, dev_u8, say

pytestmark = pytest.mark.gpu


def _run(x, p, s, N, K, G):
    st = tq.new_status()
    y = tq.gemv(dev_bf16(x), dev_u8(p), dev_f16bits(s), N, K, G, status=st)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(st.item())


@pytest.mark.parametrize("M,K", [(1, 256), (1, 8192), (4, 256), (4, 8192)])
def test_inf_activation_sets_no_flag(M, K):
    N, G = 96, 64
    w = inputs.normal_bf16(370 + K, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    x = inputs.activation(371, M, K)
    x[:, 5] = 0x7F80                          # +Inf in every activation row
    say("status word: Inf activation M=%d K=%d" % (M, K))
    y, st = _run(x, p, s, N, K, G)
    assert st == 0, st
    assert not np.isfinite(y).any()           # Inf * (+-1 or 0) summed: Inf or NaN
    # the same call with one invalid byte in row 40 sets the flag
    p2 = p.copy()
    p2[40, 3] = 251
    _, st = _run(x, p2, s, N, K, G)
    assert st == tq.DEV_INVALID_BYTE, st


@pytest.mark.parametrize("M,K", [(1, 1024), (1, 8192), (4, 1024)])
def test_overflowing_sums_set_no_flag(M, K):
    """Every code +1 (byte 242), scale 1: the first half of x is +3e38, the
    second half -3e38, so partial sums overflow to +Inf and -Inf, whose sum
    is NaN; no byte is invalid."""
    N, G = 64, 64
    B = 13
    p = np.full((N, (K // G) * B), 242, np.uint8)
    s = np.full((N, K // G), 0x3C00, np.uint16)  # fp16 1.0
    big = inputs.f32_to_bf16_bits(np.array([3e38], np.float32))[0]
    x = np.empty((M, K), np.uint16)
    x[:, :K // 2] = big
    x[:, K // 2:] = big | 0x8000
    say("status word: overflowing sums M=%d K=%d" % (M, K))
    y, st = _run(x, p, s, N, K, G)
    assert st == 0, st
    assert not np.isfinite(y).any()
    p[N - 1, -1] = 243
    _, st = _run(x, p, s, N, K, G)
    assert st == tq.DEV_INVALID_BYTE, st
