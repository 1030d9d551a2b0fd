"""Batched quantize/pack, QAT forward and unpack: every output equals its
single call and the CPU oracle, bit for bit, over one and two launches
(precisit "pack-unpack-run" README: codec.py description and scale rule;
Avenue README: BitNet-style training)."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import dev_bf16, host_u16, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,G,count", [(96, 320, 64, 70), (250, 1024, 128, 3),
                                         (3584, 1024, 128, 2), (64, 3584, 128, 65)])
def test_batched_match_single_calls_and_oracle(N, K, G, count):
    import torch
    import ternary_weight_only_amd as tq
    mats = [inputs.normal_bf16(600 + i, (N, K), 0.02) for i in range(count)]
    # one planted NaN and one overflow group, so status bits travel too
    mats[count // 2] = mats[count // 2].copy()
    mats[count // 2][1, 3] = 0x7FC0
    mats[-1] = mats[-1].copy()
    mats[-1][0, :G] = 0x7F00
    wd = [dev_bf16(m) for m in mats]
    say("batched quantize/fake/unpack W[%d,%d] G=%d count %d" % (N, K, G, count))
    st_b, st_f, st_u = tq.new_status(), tq.new_status(), tq.new_status()
    qb = tq.quantize_pack_batched(wd, G, status=st_b)
    fb = tq.fake_quantize_batched(wd, G, status=st_f, with_scales=True)
    ub = tq.unpack_batched([p for p, _ in qb], N, K, G, status=st_u)
    torch.cuda.synchronize()
    assert int(st_b.item()) == int(st_f.item()) == 1 | 2
    assert int(st_u.item()) == 0
    for i, m in enumerate(mats):
        p_ref, s_ref, _ = oracle.quantize_pack(m, G)
        f_ref, fs_ref, _ = oracle.fake_quantize(m, G)
        c_ref, _ = oracle.unpack(p_ref, N, K, G)
        p, s = qb[i]
        assert np.array_equal(p.cpu().numpy(), p_ref), "packed %d" % i
        assert np.array_equal(host_u16(s), s_ref), "scales %d" % i
        assert np.array_equal(host_u16(fb[i][0]), f_ref), "w_hat %d" % i
        assert np.array_equal(host_u16(fb[i][1]), fs_ref), "fake scales %d" % i
        assert np.array_equal(ub[i].cpu().numpy(), c_ref), "codes %d" % i
        if i in (0, count - 1):
            p1, s1 = tq.quantize_pack(wd[i], G)
            assert torch.equal(p1, p) and torch.equal(s1.view(torch.int16), s.view(torch.int16))
            assert torch.equal(tq.fake_quantize(wd[i], G).view(torch.int16),
                               fb[i][0].view(torch.int16))
            assert torch.equal(tq.unpack(p, N, K, G), ub[i])


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("offset", [0, 1, 2, 3])
def test_unpack_random_bytes_any_alignment(G, offset):
    """Random bytes over 0..255 (invalid ones and every padding pattern),
    packed data at each alignment, codes 16-byte and only 8-byte aligned;
    a small matrix (one item per thread) and 4096 x 1024."""
    import torch
    import ternary_weight_only_amd as tq
    rng = np.random.default_rng(700 + G + offset)
    for N, K in ((37, 5 * G), (4096, 1024)):
        B = (G + 4) // 5
        p = rng.integers(0, 256, size=(N, (K // G) * B)).astype(np.uint8)
        if N > 100:  # valid bytes (random padding trits), one invalid byte at the end
            p = rng.integers(0, 243, size=p.shape).astype(np.uint8)
            p[-1, -1] = 250
        flat = p.reshape(-1)
        buf = torch.zeros(flat.size + 8, dtype=torch.uint8, device="cuda")
        pd = buf[offset:offset + flat.size]
        pd.copy_(torch.from_numpy(flat))
        ref, st_ref = oracle.unpack(p, N, K, G)
        for c_off in (0, 8):
            cb = torch.empty(N * K + 16, dtype=torch.int8, device="cuda")
            cd = cb[c_off:c_off + N * K].view(N, K)
            st = tq.new_status()
            say("unpack random bytes N=%d K=%d G=%d packed offset %d codes offset %d"
                % (N, K, G, offset, c_off))
            tq.unpack(pd, N, K, G, status=st, out=cd)
            torch.cuda.synchronize()
            assert np.array_equal(cd.cpu().numpy(), ref), (N, K, c_off)
            assert int(st.item()) == st_ref
