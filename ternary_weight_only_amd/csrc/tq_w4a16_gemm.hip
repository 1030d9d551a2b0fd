// tq_w4a16_gemm.hip -- W4A16 matmul for any number of activation rows on the
// matrix cores (gfx950): y[M,N] = bf16_rne(x[M,K] * W_hat^T), W_hat = q*s + b.
//
// tiny-llm "Week 2 Day 3: Quantize the Model": the stored format
// ("Group-Wise Affine Quantization", "Packed Storage Layout": eight 4-bit
// codes a uint32, the first in the low nibble; a bf16 scale and bias per
// group), the rearranged per-group sum s * sum(x q) + b * sum(x)
// ("Mathematical Formulation") accumulated in fp32 and rounded once to bf16
// ("Computation Flow"), and the dispatch by the number of rows ("GPU
// Dispatch": a matrix-vector schedule for few rows, a matrix schedule above;
// here BM = 16 rows per block for M <= 16, 64 above).
//
// Block: 4 waves; wave w computes a BM x 32 tile of y (columns n0 + 32w ..
// n0 + 32w + 31) with v_mfma_f32_16x16x32_bf16.  A launch takes up to 64
// same-shaped problems, one per grid z index.  Per 32-wide k step, lane
// (j, q) of a wave:
//   * loads the uint32 of eight codes of W row n0 + 32w + 16t + j at k + 8q
//     (t = 0, 1) and turns each code into its exact bf16 value (the B
//     fragment: codes 0..15 need no rounding);
//   * loads eight activations x[m][k + 8q ..] of row m0 + 16a + j (the A
//     fragment; rows past M read as zero).
// Per group, one chain of MFMAs gives sum(x q) per (m, n) and a second chain
// against an all-ones B fragment gives sum(x) per m (the bias term's factor,
// in the output layout); at the group's end acc += s * sum(x q) + b * sum(x)
// in fp32.  Products x * q are exact in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kTN = 2;         // 16-column MFMA tiles per wave
constexpr int kBN = 4 * 16 * kTN;  // columns per block: 128
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kMaxBatch = 64;  // problems per launch (2.5 KB of kernel arguments)

// Up to kMaxBatch same-shaped problems per launch, passed by value; the
// grid's z index is the problem.
struct W4Batch {
  const uint16_t *x[kMaxBatch];
  const uint32_t *packed[kMaxBatch];
  const uint16_t *scales[kMaxBatch];
  const uint16_t *biases[kMaxBatch];
  uint16_t *y[kMaxBatch];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Eight 4-bit codes (code i in bits 4i..4i+3) -> their bf16 values in k
// order.  Each code becomes an fp32 integer (exact), whose high half is its
// bf16 value; a v_perm joins two high halves.
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  uint32_t p[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float f0 = (float)((lo >> (8 * b)) & 0xFFu);  // code 2b
    const float f1 = (float)((hi >> (8 * b)) & 0xFFu);  // code 2b + 1
    p[b] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8, u32x4{p[0], p[1], p[2], p[3]});
}

template <int G, int TM>
__global__ __launch_bounds__(kThreads) void w4a16_mfma_kernel(const W4Batch args, int M, int N,
                                                              int K) {
  const int pi = (int)blockIdx.z;
  const uint16_t *__restrict__ x = args.x[pi];
  const uint32_t *__restrict__ packed = args.packed[pi];
  const uint16_t *__restrict__ scales = args.scales[pi];
  const uint16_t *__restrict__ biases = args.biases[pi];
  uint16_t *__restrict__ y = args.y[pi];
  constexpr int BM = 16 * TM;
  constexpr int KS = G / 32;  // k steps per group
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * kBN + wv * 16 * kTN;
  const int m0 = blockIdx.y * BM;
  const int nG = K / G;
  const int kw = K / 8;  // code words per row

  // rows past M or N lie past the buffers' ranges and read as zero
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(packed, (uint32_t)N * (uint32_t)kw * 4u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales, (uint32_t)N * (uint32_t)nG * 2u);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(biases, (uint32_t)N * (uint32_t)nG * 2u);

  uint32_t xoff[TM], poff[kTN], soff[kTN];
#pragma unroll
  for (int a = 0; a < TM; ++a) {
    const int m = m0 + 16 * a + j;
    xoff[a] = m < M ? ((uint32_t)m * (uint32_t)K + 8u * (uint32_t)q) * 2u : kOutOfRange;
  }
#pragma unroll
  for (int t = 0; t < kTN; ++t) {
    const int n = n0 + 16 * t + j;
    poff[t] = n < N ? ((uint32_t)n * (uint32_t)kw + (uint32_t)q) * 4u : kOutOfRange;
    soff[t] = n < N ? (uint32_t)n * (uint32_t)nG * 2u : kOutOfRange;
  }
  const bf16x8 ones = __builtin_bit_cast(
      bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  f32x4 acc[TM][kTN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < kTN; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = 0; g < nG; ++g) {
    // the group's loads first: codes, activations, scale and bias
    uint32_t wd[KS][kTN];
    u32x4 xa[KS][TM];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t kk = (uint32_t)(g * G + 32 * s);
#pragma unroll
      for (int t = 0; t < kTN; ++t)
        wd[s][t] = __builtin_amdgcn_raw_buffer_load_b32(
            rp, poff[t] == kOutOfRange ? kOutOfRange : poff[t] + (kk / 8u) * 4u, 0, 0);
#pragma unroll
      for (int a = 0; a < TM; ++a)
        xa[s][a] = __builtin_amdgcn_raw_buffer_load_b128(
            rx, xoff[a] == kOutOfRange ? kOutOfRange : xoff[a] + kk * 2u, 0, 0);
    }
    float sc[kTN], bi[kTN];
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      const uint32_t o = soff[t] == kOutOfRange ? kOutOfRange : soff[t] + 2u * (uint32_t)g;
      sc[t] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, o, 0, 0));
      bi[t] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rb, o, 0, 0));
    }
    f32x4 part[TM][kTN], xs[TM];
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      xs[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kTN; ++t) part[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 bq[kTN];
#pragma unroll
      for (int t = 0; t < kTN; ++t) bq[t] = codes_to_bf16(wd[s][t]);
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, xa[s][a]);
#pragma unroll
        for (int t = 0; t < kTN; ++t)
          part[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[t], part[a][t], 0, 0, 0);
        xs[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ones, xs[a], 0, 0, 0);
      }
    }
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int t = 0; t < kTN; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[a][t][r] = fmaf(sc[t], part[a][t][r], fmaf(bi[t], xs[a][r], acc[a][t][r]));
  }

  // lane (j, q) holds rows 4q .. 4q+3 of column j of each 16 x 16 tile
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      const int n = n0 + 16 * t + j;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * a + 4 * q + r;
        if (m < M) y[(int64_t)m * N + n] = f32_to_bf16_rne(acc[a][t][r]);
      }
    }
}

template <int G, int TM>
void launch_tm(const W4Batch &args, int count, int64_t M, int64_t N, int64_t K,
               hipStream_t stream) {
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + 16 * TM - 1) / (16 * TM)),
                  (unsigned)count);
  hipLaunchKernelGGL((w4a16_mfma_kernel<G, TM>), grid, dim3(kThreads), 0, stream, args, (int)M,
                     (int)N, (int)K);
}

template <int G>
void launch_g(const W4Batch &args, int count, int64_t M, int64_t N, int64_t K,
              hipStream_t stream) {
  if (M <= 16) launch_tm<G, 1>(args, count, M, N, K, stream);
  else if (M <= 32) launch_tm<G, 2>(args, count, M, N, K, stream);
  else launch_tm<G, 4>(args, count, M, N, K, stream);
}

}  // namespace

bool w4a16_mfma_supported(int64_t M, int64_t N, int64_t K, int G) {
  // 32-bit buffer offsets: x is M*K*2 bytes, the codes N*K/2, scales N*(K/G)*2
  return (G == 64 || G == 128) && M >= 1 && N >= 1 && K >= G && K % G == 0 &&
         M * K * 2 < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31) &&
         (N + kBN) < (int64_t(1) << 30) && M <= int64_t(65535) * 64;  // grid.y <= 65535
}

void launch_w4a16_mfma_batched(int count, const uint16_t *const *xs,
                               const uint32_t *const *packeds, const uint16_t *const *scales,
                               const uint16_t *const *biases, int64_t M, int64_t N, int64_t K,
                               int G, uint16_t *const *ys, hipStream_t stream) {
  for (int i0 = 0; i0 < count; i0 += kMaxBatch) {
    const int n = count - i0 < kMaxBatch ? count - i0 : kMaxBatch;
    W4Batch args = {};
    for (int i = 0; i < n; ++i) {
      args.x[i] = xs[i0 + i]; args.packed[i] = packeds[i0 + i]; args.scales[i] = scales[i0 + i];
      args.biases[i] = biases[i0 + i]; args.y[i] = ys[i0 + i];
    }
    if (G == 64) launch_g<64>(args, n, M, N, K, stream);
    else launch_g<128>(args, n, M, N, K, stream);
  }
}

void launch_w4a16_mfma(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                       const uint16_t *biases, int64_t M, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream) {
  launch_w4a16_mfma_batched(1, &x, &packed, &scales, &biases, M, N, K, G, &y, stream);
}

}  // namespace tq
