"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and rounds them to bf16; it contains none of
the quantization or matmul arithmetic.  Both the HIP path and the CPU oracle
consume the arrays it returns; neither side generates its own inputs.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) counter stream -> two uniforms in (0, 1] from
the top 53 bits -> Box-Muller transform in float64 -> times sigma -> float32
(round to nearest even) -> bf16 (round to nearest even).  Element i of a
stream with seed s uses counters 2*(i//2) and 2*(i//2)+1; even i takes the
cosine branch, odd i the sine branch.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, counters: np.ndarray) -> np.ndarray:
    """SplitMix64 output for the given counters (uint64 array)."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (counters.astype(np.uint64) + np.uint64(1)) * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """n standard normals (float64) of stream `seed`, elements start..start+n-1."""
    idx = np.arange(start, start + n, dtype=np.uint64)
    pair = idx // np.uint64(2)
    r1 = splitmix64(seed, pair * np.uint64(2))
    r2 = splitmix64(seed, pair * np.uint64(2) + np.uint64(1))
    u1 = ((r1 >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = ((r2 >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * np.pi * u2
    return np.where((idx & np.uint64(1)) == 0, rad * np.cos(ang), rad * np.sin(ang))


def normal_bf16(seed: int, shape, sigma: float = 1.0, chunk: int = 1 << 22,
                threads: int = 8) -> np.ndarray:
    """bf16 bit patterns (uint16 array of `shape`) of N(0, sigma^2) samples.
    Element i depends only on (seed, i), so the chunks are drawn on up to
    `threads` host threads with the same result."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)

    def fill(s):
        e = min(n, s + chunk)
        v = (normal_f64(seed, e - s, start=s) * sigma).astype(np.float32)
        out[s:e] = f32_to_bf16_bits(v)

    starts = list(range(0, n, chunk))
    if len(starts) > 1 and threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(threads, len(starts))) as ex:
            list(ex.map(fill, starts))
    else:
        for s in starts:
            fill(s)
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# The synthetic workloads (seeds fixed here; shapes follow the FFN matrices of
# a Qwen-like decoder with hidden 1024 / intermediate 3584, and an 8B-class
# dense decoder with hidden 4096 / intermediate 14336).
# ---------------------------------------------------------------------------

W_SIGMA = 0.02
X_SIGMA = 1.0


def small_matrix(K: int = 512, seed: int = 0) -> np.ndarray:
    """W[256,K] ~ N(0, 0.02) with group 0 of row 0 and the last 64-group of
    row 255 forced to zero (all-zero groups)."""
    w = normal_bf16(seed, (256, K), W_SIGMA)
    w[0, 0:64] = 0
    w[255, K - 64:K] = 0
    return w


def ffn_shapes(hidden: int = 1024, inter: int = 3584):
    """(name, N, K) of the gate, up and down projections of one FFN block."""
    return [("gate", inter, hidden), ("up", inter, hidden), ("down", hidden, inter)]


def ffn_weight(layer: int, proj: int, hidden: int = 1024, inter: int = 3584) -> np.ndarray:
    """Weights of layer `layer`, projection proj (0 gate, 1 up, 2 down)."""
    _, N, K = ffn_shapes(hidden, inter)[proj]
    return normal_bf16(1000 + 3 * layer + proj, (N, K), W_SIGMA)


def activation(seed: int, M: int, K: int) -> np.ndarray:
    """x[M,K] ~ N(0,1) as bf16 bits."""
    return normal_bf16(seed, (M, K), X_SIGMA)


def w4a16_problem(seed: int, N: int, K: int, G: int):
    """Stored W4A16 parameters of one [N,K] matrix: uniform 4-bit codes in
    uint32 words [N, K/8], and per group a bf16 scale of random sign with
    magnitude 0.01|z| + 1e-4 and a bf16 bias near -7.5 s, so that the
    reconstructed weights are centred near zero in either orientation (as
    stored checkpoints hold them).  Codes and signs come from numpy's PCG64
    seeded with `seed`; magnitudes from the SplitMix64 normal stream."""
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 1 << 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    nG = K // G
    mag = np.abs(normal_f64(seed, N * nG)).reshape(N, nG) * 0.01 + 1e-4
    sign = np.where(rng.integers(0, 2, size=mag.shape) == 1, -1.0, 1.0)
    s = f32_to_bf16_bits((sign * mag).astype(np.float32))
    b = f32_to_bf16_bits((-sign * mag * 7.5 + 0.001 * normal_f64(seed + 1, N * nG).reshape(N, nG))
                         .astype(np.float32))
    return packed, s, b


def stack_shapes(layers: int = 24):
    """(N, K) of the FFN stack's matrices, layer by layer: gate, up, down."""
    return [(N, K) for _ in range(layers) for _, N, K in ffn_shapes()]


def stack_weights(layers: int = 24, threads: int = 8):
    """The FFN stack's bf16 weights in stack_shapes() order (matrix i is
    ffn_weight(i // 3, i % 3)), generated on `threads` host threads."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda i: ffn_weight(i // 3, i % 3), range(3 * layers)))


def stack_decode_activation(i: int, K: int) -> np.ndarray:
    """The M = 1 activations of stack matrix i (seed 5000 + i)."""
    return activation(5000 + i, 1, K)


def prefill_activation(M: int, K: int) -> np.ndarray:
    """Prefill activations x[M,K] shared by every stack matrix of width K:
    seeds 30 (K = 1024) and 31 (K = 3584) at M = 512, 32 and 33 at M = 2048,
    and 34 + K for other M."""
    seeds = {(512, 1024): 30, (512, 3584): 31, (2048, 1024): 32, (2048, 3584): 33}
    return activation(seeds.get((M, K), 34 + K), M, K)


def dense8b_shapes():
    """(name, N, K) of the 8B-class dense FFN matrices."""
    return [("up", 14336, 4096), ("down", 4096, 14336)]


def dense8b_weight(N: int, K: int) -> np.ndarray:
    """W[N,K] ~ N(0, 0.02): seed 40 for W[14336,4096], 41 for W[4096,14336]."""
    return normal_bf16(40 if N > K else 41, (N, K), W_SIGMA)


def dense8b_activation(M: int, N: int, K: int) -> np.ndarray:
    """x[M,K] for the 8B-class matrix W[N,K]: seeds 50..52 (W[14336,4096]) or
    53..55 (W[4096,14336]) for M = 1, 4, 16; 56 + M otherwise."""
    idx = {1: 0, 4: 1, 16: 2}
    if M in idx:
        return activation((50 if N > K else 53) + idx[M], M, K)
    return activation(56 + M, M, K)
