"""Checks of the seeded input generator (SplitMix64 -> Box-Muller -> bf16)."""
import numpy as np
import torch

from ternary_weight_only_amd import inputs


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 started from state 0 (Steele, Lea, Flood 2014).
    got = inputs.splitmix64(0, np.arange(3, dtype=np.uint64))
    assert [int(v) for v in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    ours = inputs.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_normal_moments_and_chunking():
    a = inputs.normal_bf16(3, (1 << 20,), 1.0, chunk=1 << 17)
    b = inputs.normal_bf16(3, (1 << 20,), 1.0)
    assert np.array_equal(a, b)
    f = inputs.bf16_bits_to_f32(a).astype(np.float64)
    assert abs(f.mean()) < 5e-3 and abs(f.std() - 1) < 5e-3
    w = inputs.bf16_bits_to_f32(inputs.normal_bf16(4, (1 << 18,), 0.02)).astype(np.float64)
    assert abs(w.std() - 0.02) < 2e-4


def test_workload_shapes():
    shapes = inputs.ffn_shapes()
    assert shapes == [("gate", 3584, 1024), ("up", 3584, 1024), ("down", 1024, 3584)]
    assert 24 * sum(n * k for _, n, k in shapes) == 264241152
    w = inputs.small_matrix()
    assert w.shape == (256, 512) and not w[0, :64].any() and not w[255, -64:].any()
