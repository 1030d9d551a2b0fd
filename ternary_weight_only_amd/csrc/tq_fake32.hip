// tq_fake32.hip -- the QAT forward from fp32 latent weights on gfx950:
//   w_hat[n,k] = c[n,k] * s[n,k/G]   (fp32, exact: s is an fp16 value)
// with the group scale s = RNE_fp16(mean of |w| over the group, from the
// exact sum of the fp32 magnitudes) and the codes c = sign(w) where
// |w| > s/2, else 0 (precisit "pack-unpack-run" README, codec.py description
// and scale-rule paragraph).  Avenue README, introduction: BitNet-style
// training keeps full-precision latent weights and ternarizes them in the
// forward pass; the backward pass is straight-through and needs no kernel.
//
// A wave takes chunks of 512 consecutive weights (512/G whole groups); each
// lane loads 8 fp32 with two 16-byte loads and G/8 lanes share a group.
//   * Scale, fast path: the magnitudes are summed in fp32, 8 in order per
//     lane, then a butterfly over the group's lanes (every step pairs lanes
//     symmetrically, so all of them end with the same sum S_hat).  At most
//     7 + log2(G/8) <= 11 rounded additions of non-negative terms lie on any
//     path, so |S_hat - S| <= 11 * 2^-24 * S, plus G * 2^-126 should
//     subnormals be flushed.  With E = 2^-19 S_hat + 2^-118 the exact sum
//     lies in [S_hat - E, S_hat + E]; when both ends divided by G round to
//     the same fp16 value, so does the exact mean (rounding is monotonic).
//   * Exact path, for the groups whose interval holds an fp16 rounding
//     boundary: the group's magnitudes are summed as a 320-bit integer in
//     units of 2^-149 (8 per lane, then a butterfly over the group's lanes,
//     whose integer additions are exact in any order) and the mean is
//     rounded once.
//   * Codes compare the magnitudes' bit patterns with those of s/2 (exact);
//     a group with an Inf/NaN weight or a mean that rounds to >= 65520 is
//     flagged and gets w_hat = +0.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxBlocks = 16384;  // blocks of one launch, over all its problems
constexpr int kMaxBatch = 64;      // problems per launch

struct Fake32Batch {
  const float *w[kMaxBatch];
  float *w_hat[kMaxBatch];
  uint16_t *scales[kMaxBatch];
};

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, kWave);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = shfl_xor_u32((uint32_t)v, mask);
  const uint32_t hi = shfl_xor_u32((uint32_t)(v >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}

// fp16 bits of the mean of an exact sum A * 2^-149 (A: 320-bit integer,
// little-endian limbs) over 2^t terms, rounded once to nearest, ties to
// even; sets *ovf and returns 0x7C00 when it rounds to >= 65520.
__device__ __forceinline__ uint32_t f16_of_exact_sum(const uint64_t (&A)[5], int t, bool *ovf) {
  int L = -1;
#pragma unroll
  for (int i = 4; i >= 0; --i)
    if (L < 0 && A[i]) L = 64 * i + 63 - __clzll((long long)A[i]);
  *ovf = false;
  if (L < 0) return 0;
  auto limb = [&](int i) -> uint64_t { return (i >= 0 && i < 5) ? A[i] : 0ull; };
  auto bits_at = [&](int pos) -> uint64_t {  // bits [pos, pos + 13), pos >= 0
    const int i = pos >> 6, o = pos & 63;
    const uint64_t v = (limb(i) >> o) | (o ? limb(i + 1) << (64 - o) : 0ull);
    return v & 0x1FFFull;
  };
  auto any_below = [&](int pos) -> bool {  // any bit below position pos >= 0
    const int i = pos >> 6, o = pos & 63;
    bool any = o ? (limb(i) & ((1ull << o) - 1)) != 0 : false;
    for (int k = 0; k < i && k < 5; ++k) any |= A[k] != 0;
    return any;
  };
  auto rne_at = [&](int d) -> uint64_t {  // RNE(A / 2^d), d >= 1, result < 2^13
    const uint64_t q = bits_at(d);
    const bool half = ((limb((d - 1) >> 6) >> ((d - 1) & 63)) & 1ull) != 0;
    const bool sticky = any_below(d - 1);
    return q + ((half && (sticky || (q & 1))) ? 1 : 0);
  };
  // the mean in units of the fp16 subnormal step 2^-24 is A / 2^(125 + t)
  const int r = 125 + t;
  if (L < r + 10) return (uint32_t)rne_at(r);  // below 1024 steps
  const int k = L - r - 10;                     // mean in [2^(10+k), 2^(11+k)) steps
  if (k >= 30) { *ovf = true; return 0x7C00; }
  const uint32_t bits = ((uint32_t)k << 10) + (uint32_t)rne_at(L - 10);
  if (bits >= 0x7C00) { *ovf = true; return 0x7C00; }
  return bits;
}

// A += v, both 320-bit
__device__ __forceinline__ void add320(uint64_t (&A)[5], const uint64_t (&v)[5]) {
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t s1 = A[i] + v[i];
    const uint64_t c1 = s1 < v[i];
    const uint64_t s2 = s1 + carry;
    carry = c1 + (s2 < s1);
    A[i] = s2;
  }
}

// A += |w| in units of 2^-149.  A finite magnitude u is sig * 2^(e - 149):
// normal (E = u >> 23 >= 1) sig = 2^23 + m, e = E - 1; subnormal sig = m, e = 0.
__device__ __forceinline__ void add_mag(uint64_t (&A)[5], uint32_t u) {
  const uint32_t E = u >> 23, m = u & 0x7FFFFFu;
  const uint64_t sig = E ? (1ull << 23) + m : m;
  const int e = E ? (int)E - 1 : 0;
  const int li = e >> 6, off = e & 63;
  uint64_t v[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t lo = sig << off, hi = off ? (sig >> (64 - off)) : 0ull;
    v[i] = i == li ? lo : (i == li + 1 ? hi : 0ull);
  }
  add320(A, v);
}

template <int G>
__global__ __launch_bounds__(kBlock) void fake_quantize_f32_kernel(const Fake32Batch args,
                                                                   int64_t total_groups,
                                                                   int32_t *__restrict__ d_status) {
  const float *__restrict__ w = args.w[blockIdx.y];
  float *__restrict__ w_hat = args.w_hat[blockIdx.y];
  uint16_t *__restrict__ scales = args.scales[blockIdx.y];
  constexpr int LPG = G / 8;    // lanes per group
  constexpr int GPC = 512 / G;  // groups per chunk
  constexpr int LOG2G = (G == 64) ? 6 : 7;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane % LPG;
  const int qg = lane / LPG;
  const int64_t nchunks = (total_groups + GPC - 1) / GPC;

  for (int64_t base = (int64_t)blockIdx.x * kWavesPerBlock; base < nchunks;
       base += (int64_t)gridDim.x * kWavesPerBlock) {
    const int64_t chunk = base + wv;
    const int64_t gi = chunk * GPC + qg;
    const bool active = chunk < nchunks && gi < total_groups;

    uint32_t u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active) {
      const uint4 a = *reinterpret_cast<const uint4 *>(w + gi * G + sub * 8);
      const uint4 b = *reinterpret_cast<const uint4 *>(w + gi * G + sub * 8 + 4);
      u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w;
      u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
    }

    float acc = 0.f;
    uint32_t maxmag = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t mag = u[i] & 0x7FFFFFFFu;
      maxmag = mag > maxmag ? mag : maxmag;
      acc += __uint_as_float(mag);
    }
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) {
      acc += __uint_as_float(shfl_xor_u32(__float_as_uint(acc), m));
      const uint32_t o = shfl_xor_u32(maxmag, m);
      maxmag = o > maxmag ? o : maxmag;
    }
    uint32_t sbits = 0;
    int flags = 0;
    bool slow = false;
    if (maxmag >= 0x7F800000u) {  // an Inf or NaN weight
      sbits = 0x7E00;
      flags = kDevNonfinite;
    } else {
      const float E = fmaf(acc, 0x1p-19f, 0x1p-118f);
      constexpr float kInvG = 1.0f / G;
      const uint32_t qlo = __half_as_ushort(__float2half_rn(fmaxf(acc - E, 0.f) * kInvG));
      const uint32_t qhi = __half_as_ushort(__float2half_rn((acc + E) * kInvG));
      if (qlo == qhi) {
        sbits = qlo;
        if (sbits >= 0x7C00u) {
          sbits = 0x7C00;
          flags = kDevScaleOverflow;
        }
      } else {
        slow = true;
      }
    }
    // Exact path, taken by the whole wave when one of its groups needs it
    // (its shuffles need every lane): each lane sums its 8 magnitudes as a
    // 320-bit integer, the group's lanes add theirs in a butterfly, and
    // every lane rounds the exact mean once.
    if (__any(slow)) {
      uint64_t A[5] = {0, 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) add_mag(A, u[i] & 0x7FFFFFFFu);
#pragma unroll
      for (int m = 1; m < LPG; m <<= 1) {
        uint64_t o[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) o[i] = shfl_xor_u64(A[i], m);
        add320(A, o);
      }
      if (slow) {
        bool ovf;
        sbits = f16_of_exact_sum(A, LOG2G, &ovf);
        flags = ovf ? kDevScaleOverflow : 0;
      }
    }

    // codes: |w| > s/2 on ordered bit patterns; w_hat = +-s or +0 (c = 0,
    // s >= 0), -0 for c = -1 with s = +0; a flagged group is +0
    const float s = __half2float(__ushort_as_half((unsigned short)sbits));
    const uint32_t s_bits = __float_as_uint(s);
    const uint32_t half_bits = __float_as_uint(s * 0.5f);
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t mag = u[i] & 0x7FFFFFFFu;
      out[i] = (!flags && mag > half_bits) ? (s_bits | (u[i] & 0x80000000u)) : 0u;
    }
    if (active) {
      *reinterpret_cast<uint4 *>(w_hat + gi * G + sub * 8) = make_uint4(out[0], out[1], out[2], out[3]);
      *reinterpret_cast<uint4 *>(w_hat + gi * G + sub * 8 + 4) =
          make_uint4(out[4], out[5], out[6], out[7]);
      if (sub == 0) {
        if (scales) scales[gi] = (uint16_t)sbits;
        if (flags && d_status) atomicOr(d_status, flags);
      }
    }
  }
}

}  // namespace

void launch_fake_quantize_f32_batched(int count, const float *const *ws, int64_t N, int64_t K,
                                      int G, float *const *w_hats, uint16_t *const *scales,
                                      int32_t *d_status, hipStream_t stream) {
  const int64_t total_groups = N * (K / G);
  const int64_t chunks = (total_groups * G + 511) / 512;
  for (int i0 = 0; i0 < count; i0 += kMaxBatch) {
    const int n = count - i0 < kMaxBatch ? count - i0 : kMaxBatch;
    Fake32Batch a{};
    for (int i = 0; i < n; ++i) {
      a.w[i] = ws[i0 + i];
      a.w_hat[i] = w_hats[i0 + i];
      a.scales[i] = scales ? scales[i0 + i] : nullptr;
    }
    int64_t blocks = (chunks + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t cap = kMaxBlocks / n > 0 ? kMaxBlocks / n : 1;
    if (blocks > cap) blocks = cap;
    const dim3 grid((unsigned)blocks, (unsigned)n);
    if (G == 64)
      hipLaunchKernelGGL(fake_quantize_f32_kernel<64>, grid, dim3(kBlock), 0, stream, a,
                         total_groups, d_status);
    else
      hipLaunchKernelGGL(fake_quantize_f32_kernel<128>, grid, dim3(kBlock), 0, stream, a,
                         total_groups, d_status);
  }
}

}  // namespace tq
