"""GPU parity of the decode to bf16 (tq_dequantize) against the CPU oracle.

Bar: bit-exact bf16 patterns and status bits (precisit "pack-unpack-run"
README, codec.py description: decoding gives back c * s; screen.py
description: the decoder hands the weights back as bf16)."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import dev_f16bits, dev_u8, host_u16, say

pytestmark = pytest.mark.gpu


def gpu_dequant(packed, scales, N, K, G, offset=0):
    import torch
    import ternary_weight_only_amd as tq
    flat = np.ascontiguousarray(packed).reshape(-1)
    buf = torch.zeros(flat.size + 8, dtype=torch.uint8, device="cuda")
    pd = buf[offset:offset + flat.size]
    pd.copy_(torch.from_numpy(flat))
    st = tq.new_status()
    w = tq.dequantize(pd, dev_f16bits(scales), N, K, G, status=st)
    torch.cuda.synchronize()
    return host_u16(w), int(st.item())


def check(packed, scales, N, K, G, what, offset=0):
    got, st = gpu_dequant(packed, scales, N, K, G, offset)
    ref, st_ref = oracle.dequantize(packed, scales, N, K, G)
    bad = got != ref
    assert not bad.any(), "%s: %d of %d differ, first at %s: %#06x vs %#06x" % (
        what, int(bad.sum()), bad.size, tuple(np.argwhere(bad)[0]),
        int(got[bad][0]), int(ref[bad][0]))
    assert st == st_ref, "%s: status %d vs %d" % (what, st, st_ref)
    return st


@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (1, 128, 128), (7, 192, 64), (3, 384, 128),
                                   (256, 512, 64), (250, 1024, 128), (33, 3584, 128),
                                   (129, 320, 64)])
def test_quantized_matrices_exact(N, K, G):
    w = inputs.normal_bf16(70 + N, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    say("dequantize W[%d,%d] G=%d" % (N, K, G))
    assert check(p, s, N, K, G, "W[%d,%d] G=%d" % (N, K, G)) == 0


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("offset", [0, 1, 2, 3])
def test_every_byte_value_any_alignment_and_special_scales(G, offset):
    """Random bytes over 0..255 (invalid ones included), every padding
    pattern, packed data at each alignment, and scales of every kind: signed
    zeros, subnormals, 65504, rounding ties, Inf and NaN."""
    rng = np.random.default_rng(80 + G + offset)
    N, K = 37, 5 * G
    B = (G + 4) // 5
    p = rng.integers(0, 256, size=(N, (K // G) * B)).astype(np.uint8)
    s = rng.integers(0, 0x10000, size=(N, K // G)).astype(np.uint16)
    special = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x7BFF, 0xFBFF, 0x3C04, 0x3C0C, 0x3C05,
               0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFFFF]
    s.reshape(-1)[:len(special)] = special
    say("dequantize random bytes G=%d offset %d" % (G, offset))
    st = check(p, s, N, K, G, "random bytes G=%d offset %d" % (G, offset), offset)
    assert st == 1 | 4 | 8


@pytest.mark.parametrize("G", [64, 128])
def test_flags_one_at_a_time(G):
    N, K = 16, 4 * G
    w = inputs.normal_bf16(90, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    B = (G + 4) // 5
    bad = p.copy()
    bad[3, 5] = 250
    assert check(bad, s, N, K, G, "invalid byte") == 4
    last = p.copy()
    last.reshape(-1)[-1] = 255                    # the buffer's very last byte
    assert check(last, s, N, K, G, "invalid last byte") == 4
    pad = p.copy()
    v = int(pad[7, 2 * B - 1])                    # last byte of group 1: holds the padding
    pad[7, 2 * B - 1] = v + 81 if v < 162 else v - 81
    assert check(pad, s, N, K, G, "bad padding") == 8
    nf = s.copy()
    nf[2, 1] = 0x7E00
    assert check(p, nf, N, K, G, "NaN scale") == 1


@pytest.mark.parametrize("N,K", [(3584, 1024), (1024, 3584)])
def test_ffn_matrix_full_size(N, K):
    """A whole FFN projection of the Qwen-like stack (G=128), every element."""
    w = inputs.ffn_weight(0, 0 if K == 1024 else 2)
    assert w.shape == (N, K)
    p, s, _ = oracle.quantize_pack(w, 128)
    say("dequantize FFN W[%d,%d] G=128" % (N, K))
    assert check(p, s, N, K, 128, "FFN W[%d,%d]" % (N, K)) == 0


def test_many_passes_of_the_grid():
    """More items than one pass of the launch's grid covers (8192 x 4096,
    G=128: 4.2M items of 8 weights), every element."""
    N, K, G = 8192, 4096, 128
    w = inputs.normal_bf16(91, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    say("dequantize W[%d,%d] G=%d" % (N, K, G))
    assert check(p, s, N, K, G, "W[8192,4096]") == 0


def test_gpu_quantize_then_decode_matches_oracle_chain():
    import torch
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16
    N, K, G = 500, 2048, 128
    w = inputs.normal_bf16(92, (N, K), 0.02)
    st = tq.new_status()
    pd, sd = tq.quantize_pack(dev_bf16(w), G, status=st)
    wd = tq.dequantize(pd, sd, N, K, G, status=st)
    torch.cuda.synchronize()
    p, s, _ = oracle.quantize_pack(w, G)
    ref, _ = oracle.dequantize(p, s, N, K, G)
    assert int(st.item()) == 0
    assert np.array_equal(host_u16(wd), ref)


@pytest.mark.parametrize("N,K,G,count", [(96, 320, 64, 70), (250, 1024, 128, 3), (3584, 1024, 128, 2)])
def test_batched_matches_single_calls_and_oracle(N, K, G, count):
    """count > 64 takes two launches; each output equals its own single call
    and the oracle, bit for bit."""
    import torch
    import ternary_weight_only_amd as tq
    mats = [oracle.quantize_pack(inputs.normal_bf16(100 + i, (N, K), 0.02), G)[:2]
            for i in range(count)]
    pk = [dev_u8(p) for p, _ in mats]
    sc = [dev_f16bits(s) for _, s in mats]
    say("dequantize_batched W[%d,%d] G=%d count %d" % (N, K, G, count))
    st = tq.new_status()
    outs = tq.dequantize_batched(pk, sc, N, K, G, status=st)
    single = [tq.dequantize(p, s, N, K, G) for p, s in zip(pk, sc)]
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, (p, s) in enumerate(mats):
        ref, _ = oracle.dequantize(p, s, N, K, G)
        got = host_u16(outs[i])
        assert np.array_equal(got, ref), "problem %d differs from the oracle" % i
        assert np.array_equal(got, host_u16(single[i])), "problem %d differs from its call" % i


def test_batched_grid_stride_passes():
    """64 problems of W[2080,4096] (G=128): 1,064,960 items each, more than
    the launch's blocks per problem cover in one pass (65536 blocks over 64
    problems, 4 items per thread), so every thread strides a second time.
    All inputs hold the same matrix (distinct copies): the first output is
    checked against the oracle, the others against the first, on the device."""
    import torch
    import ternary_weight_only_amd as tq
    N, K, G, count = 2080, 4096, 128, 64
    p, s, _ = oracle.quantize_pack(inputs.normal_bf16(110, (N, K), 0.02), G)
    pd, sd = dev_u8(p), dev_f16bits(s)
    pk = [pd.clone() for _ in range(count)]
    sc = [sd.clone() for _ in range(count)]
    say("dequantize_batched W[%d,%d] G=%d count %d (grid-stride)" % (N, K, G, count))
    st = tq.new_status()
    outs = tq.dequantize_batched(pk, sc, N, K, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref, _ = oracle.dequantize(p, s, N, K, G)
    assert np.array_equal(host_u16(outs[0]), ref)
    for i in range(1, count):
        assert torch.equal(outs[i], outs[0]), "problem %d differs" % i


@pytest.mark.parametrize("N,K", [(3584, 3584), (1000, 2048)])
def test_middle_sizes_exact(N, K):
    """Launch sizes between the small and the large cases (2 and 1 items per
    thread), every element."""
    w = inputs.normal_bf16(111, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, 128)
    say("dequantize W[%d,%d] G=128" % (N, K))
    assert check(p, s, N, K, 128, "W[%d,%d]" % (N, K)) == 0
