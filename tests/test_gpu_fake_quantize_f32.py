"""GPU parity of the QAT forward from fp32 latent weights
(tq_fake_quantize_f32, tq_fake_quantize_f32_batched) against the CPU oracle:
fp32 w_hat = c * s, fp16 scales and status bits bit-exact (Avenue README,
introduction: BitNet-style training keeps full-precision latent weights;
precisit "pack-unpack-run" README: the scale and code rule)."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import host_u16, say

pytestmark = pytest.mark.gpu


def _dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def gpu_fake32(w, G):
    import torch
    import ternary_weight_only_amd as tq
    N, K = w.shape
    st = tq.new_status()
    sc = torch.empty((N, K // G), dtype=torch.float16, device="cuda")
    w_hat = tq.fake_quantize_f32(_dev_f32(w), G, status=st, scales_out=sc)
    torch.cuda.synchronize()
    return w_hat.cpu().numpy(), host_u16(sc), int(st.item())


def check(w, G, what):
    got, sc, st = gpu_fake32(w, G)
    ref, sc_ref, st_ref = oracle.fake_quantize_f32(w, G)
    g, r = got.view(np.uint32), ref.view(np.uint32)
    bad = g != r
    assert not bad.any(), "%s: %d of %d differ, first at %s: %#010x vs %#010x" % (
        what, int(bad.sum()), bad.size, tuple(np.argwhere(bad)[0]), int(g[bad][0]),
        int(r[bad][0]))
    assert np.array_equal(sc, sc_ref), what
    assert st == st_ref, "%s: status %d vs %d" % (what, st, st_ref)
    return st


def _wide(rng, shape, emin, emax):
    n = int(np.prod(shape))
    sign = rng.integers(0, 2, n).astype(np.uint32) << 31
    e = rng.integers(emin, emax + 1, n).astype(np.uint32) << 23
    m = rng.integers(0, 1 << 23, n).astype(np.uint32)
    return (sign | e | m).view(np.float32).reshape(shape)


@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (1, 128, 128), (7, 192, 64), (256, 512, 64),
                                   (33, 1024, 128), (3, 4096, 128)])
def test_normal_matrices_exact(N, K, G):
    rng = np.random.default_rng(900 + N + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    say("fake32 N=%d K=%d G=%d" % (N, K, G))
    assert check(w, G, "N=%d K=%d G=%d" % (N, K, G)) == 0


@pytest.mark.parametrize("G", [64, 128])
def test_wide_exponents_and_subnormals_exact(G):
    """Random fp32 bit patterns over exponents -149 .. +15 (the exact path
    runs for many groups), and groups of subnormals only (scale 0)."""
    rng = np.random.default_rng(910 + G)
    check(_wide(rng, (64, 4 * G), 0, 141), G, "wide exponents")
    check(_wide(rng, (8, 2 * G), 0, 0), G, "subnormals")


@pytest.mark.parametrize("G", [64, 128])
def test_means_on_fp16_midpoints_exact(G):
    """Groups whose exact mean is an fp16 midpoint, plus or minus a few fp32
    steps of one weight: the fast interval straddles the boundary, so the
    exact path decides each one."""
    rng = np.random.default_rng(920 + G)
    rows = []
    for i in range(96):
        k = int(rng.integers(-20, 12))               # midpoint exponent
        mid = (1.0 + (2 * int(rng.integers(0, 512)) + 1) * 2.0 ** -11) * 2.0 ** k
        g = np.full(G, mid, np.float64)
        g[::2] *= -1.0                              # signs do not change the mean
        j = int(rng.integers(0, G))
        g32 = g.astype(np.float32)
        d = int(rng.integers(-2, 3))
        if d:
            u = g32[j:j + 1].view(np.uint32)
            u += np.uint32(abs(d)) if d > 0 else np.uint32(0)
            if d < 0:
                u -= np.uint32(-d)
        rows.append(g32)
    check(np.stack(rows), G, "midpoints")


def test_flags_exact():
    G = 64
    w = np.tile(np.array([0.01, -0.01], np.float32), (5, 2 * G // 2))
    w[0, 3] = np.nan
    w[1, G + 9] = np.inf
    w[2, :G] = np.tile(np.array([3.0e38, -3.0e38], np.float32), G // 2)
    w[3, G:] = np.tile(np.array([1e-40, -1e-40], np.float32), G // 2)
    st = check(w, G, "flags")
    assert st == 1 | 2


def test_ffn_matrix_full_size():
    """One FFN matrix W[3584,1024] of fp32 weights ~N(0, 0.02), both G."""
    rng = np.random.default_rng(930)
    w = (rng.standard_normal((3584, 1024)) * 0.02).astype(np.float32)
    for G in (64, 128):
        say("fake32 FFN G=%d" % G)
        assert check(w, G, "FFN G=%d" % G) == 0


def test_batched_equals_single_and_gradient():
    """Batched launches (70 matrices: two launches) equal single calls bit
    for bit; FakeQuantize on an fp32 tensor runs this forward and passes the
    gradient straight through."""
    import torch
    import ternary_weight_only_amd as tq
    rng = np.random.default_rng(940)
    ws = [(rng.standard_normal((16, 256)) * 0.02).astype(np.float32) for _ in range(70)]
    dws = [_dev_f32(w) for w in ws]
    st = tq.new_status()
    outs = tq.fake_quantize_f32_batched(dws, 128, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, (w, o) in enumerate(zip(ws, outs)):
        ref, _, _ = oracle.fake_quantize_f32(w, 128)
        assert np.array_equal(o.cpu().numpy().view(np.uint32), ref.view(np.uint32)), i
    x = dws[0].clone().requires_grad_(True)
    y = tq.FakeQuantize.apply(x, 128)
    assert y.dtype == torch.float32
    g = torch.randn_like(y)
    y.backward(g)
    torch.cuda.synchronize()
    assert torch.equal(x.grad, g)
    ref, _, _ = oracle.fake_quantize_f32(ws[0], 128)
    assert np.array_equal(y.detach().cpu().numpy().view(np.uint32), ref.view(np.uint32))
