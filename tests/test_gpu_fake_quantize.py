"""GPU parity of the QAT forward (tq_fake_quantize) against the CPU oracle,
and its straight-through gradient.  Bar: bit-exact bf16 w_hat, fp16 scales
and status bits (Avenue README: BitNet-style training on latent weights;
precisit "pack-unpack-run" README: the scale and code rule)."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import dev_bf16, host_u16, say
from tests.test_gpu_parity import _bf16, _random_finite_bf16

pytestmark = pytest.mark.gpu


def gpu_fake(w_bits, G, with_scales=True):
    import torch
    import ternary_weight_only_amd as tq
    N, K = w_bits.shape
    st = tq.new_status()
    sc = torch.empty((N, K // G), dtype=torch.float16, device="cuda") if with_scales else None
    w_hat = tq.fake_quantize(dev_bf16(w_bits), G, status=st, scales_out=sc)
    torch.cuda.synchronize()
    return host_u16(w_hat), (host_u16(sc) if with_scales else None), int(st.item())


def check(w_bits, G, what, with_scales=True):
    got, sc, st = gpu_fake(w_bits, G, with_scales)
    ref, sc_ref, st_ref = oracle.fake_quantize(w_bits, G)
    bad = got != ref
    assert not bad.any(), "%s: %d of %d differ, first at %s: %#06x vs %#06x" % (
        what, int(bad.sum()), bad.size, tuple(np.argwhere(bad)[0]), int(got[bad][0]),
        int(ref[bad][0]))
    if with_scales:
        assert np.array_equal(sc, sc_ref), what
    assert st == st_ref, "%s: status %d vs %d" % (what, st, st_ref)
    return st


@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (1, 128, 128), (7, 192, 64), (256, 512, 64),
                                   (250, 1024, 128), (33, 3584, 128), (129, 320, 64)])
def test_matrices_exact(N, K, G):
    w = inputs.normal_bf16(500 + N, (N, K), 0.02)
    say("fake_quantize W[%d,%d] G=%d" % (N, K, G))
    assert check(w, G, "W[%d,%d] G=%d" % (N, K, G)) == 0


@pytest.mark.parametrize("G", [64, 128])
def test_stress_groups_exact(G):
    """Exponents over ~140 binades, bf16 subnormals, fp16 midpoints, overflow
    and non-finite groups (which give +0 and their flags)."""
    rng = np.random.default_rng(501)
    rows = [_random_finite_bf16(rng, 64 * G, 0, 140).reshape(64, G),
            _random_finite_bf16(rng, 64 * G, 90, 120).reshape(64, G),
            _random_finite_bf16(rng, 64 * G, 0, 10).reshape(64, G)]
    special = np.zeros((6, G), np.uint16)
    half = G // 2
    special[0, :half] = _bf16(2.0)
    special[0, half] = _bf16(G * 2.0 ** -11)      # mean on an fp16 midpoint
    special[1, :] = _bf16(7e4)                   # overflow
    special[2, :] = _bf16(2.0 ** -30)            # underflow to s = 0
    special[3, :] = inputs.normal_bf16(502, (G,), 0.02)
    special[3, 3] = 0x7FC1                       # NaN
    special[4, :] = _bf16(1.0)
    special[4, 7] = 0xFF80                       # -inf
    special[5, :] = _bf16(65504.0 / 2)
    w = np.concatenate(rows + [special])
    say("fake_quantize stress G=%d" % G)
    assert check(w, G, "stress G=%d" % G) == 1 | 2
    assert check(w, G, "stress G=%d, no scales" % G, with_scales=False) == 1 | 2


@pytest.mark.parametrize("proj", [0, 2])
def test_ffn_matrix_full_size_and_pack_decode_agree(proj):
    """A whole FFN projection (G=128): every element against the oracle, and
    against tq_quantize_pack followed by tq_dequantize on the GPU."""
    import torch
    import ternary_weight_only_amd as tq
    w = inputs.ffn_weight(1, proj)
    N, K = w.shape
    say("fake_quantize FFN W[%d,%d]" % (N, K))
    assert check(w, 128, "FFN W[%d,%d]" % (N, K)) == 0
    wd = dev_bf16(w)
    p, s = tq.quantize_pack(wd, 128)
    d = tq.dequantize(p, s, N, K, 128)
    f = tq.fake_quantize(wd, 128)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), f.view(torch.int16))


def test_straight_through_gradient():
    import torch
    import ternary_weight_only_amd as tq
    w = dev_bf16(inputs.normal_bf16(503, (64, 256), 0.02)).requires_grad_(True)
    g = dev_bf16(inputs.normal_bf16(504, (64, 256), 1.0))
    w_hat = tq.FakeQuantize.apply(w, 64)
    ref, _, _ = oracle.fake_quantize(host_u16(w.detach()), 64)
    assert np.array_equal(host_u16(w_hat.detach()), ref)
    (w_hat * g).sum().backward()
    torch.cuda.synchronize()
    assert w.grad is not None and torch.equal(w.grad.view(torch.int16), g.view(torch.int16))
