// tq_gemm.hip -- prefill matmul for gfx950: packed ternary tiles are decoded
// into LDS as bf16 codes (exact), multiplied with bf16 activations on MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate) one K-group at a time, and each
// group's fp32 partial is scaled by its fp16 scale in fp32.
//
// y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
// (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation";
// prefill reuses each weight tile across many rows, "Revisit the Decode
// Roofline").
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int BM = 64;  // activation rows per block (16 per wave)
constexpr int BN = 64;  // weight rows per block (4 MFMA column tiles)

// MFMA 16x16x32 operand layout used below: lane l holds A[l%16][8*(l/16)+e]
// and B[8*(l/16)+e][l%16] for e = 0..7; the result D[i][j] sits in lane
// j + 16*(i/4), element i%4.
template <int G>
__global__ __launch_bounds__(kBlock) void gemm_tile_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scales, int64_t M, int64_t N, int64_t K, float *__restrict__ y,
    int32_t *__restrict__ d_status) {
  constexpr int B = bytes_per_group(G);
  constexpr int LDC = G + 8;  // padded LDS row (bf16 elements)
  __shared__ __align__(16) uint16_t codes_s[BN * LDC];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t nG = K / G;
  const int64_t arow = m0 + wv * 16 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  int flags = 0;

  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t g = 0; g < nG; ++g) {
    __syncthreads();
    for (int idx = tid; idx < BN * B; idx += kBlock) {
      const int r = idx / B, b = idx % B;
      const int64_t n = n0 + r;
      uint32_t v = n < N ? packed[(n * nG + g) * B + b] : 121u;
      if (v >= 243u) { flags |= kDevInvalidByte; v = 121u; }
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const uint32_t d = v % 3u;
        v /= 3u;
        const int pos = 5 * b + i;
        if (pos < G) codes_s[r * LDC + pos] = d == 0u ? 0xBF80u : (d == 2u ? 0x3F80u : 0u);
      }
    }
    float s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t n = n0 + 16 * t + (lane & 15);
      s[t] = n < N ? __half2float(__ushort_as_half(scales[n * nG + g])) : 0.f;
    }
    __syncthreads();

    f32x4 part[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) part[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < G; kk += 32) {
      bf16x8 a;
      if (arow < M) {
        a = *reinterpret_cast<const bf16x8 *>(x + arow * K + g * G + kk + kq);
      } else {
        const uint4 z = make_uint4(0, 0, 0, 0);
        a = *reinterpret_cast<const bf16x8 *>(&z);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 bv =
            *reinterpret_cast<const bf16x8 *>(&codes_s[(16 * t + (lane & 15)) * LDC + kk + kq]);
        part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, part[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(s[t], part[t][r], acc[t][r]);
  }

#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t n = n0 + 16 * t + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wv * 16 + 4 * (lane >> 4) + r;
      if (m < M && n < N) y[m * N + n] = acc[t][r];
    }
  }
  if (flags && d_status) atomicOr(d_status, flags);
}

}  // namespace

void launch_gemm(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t M,
                 int64_t N, int64_t K, int G, float *y, int32_t *d_status, hipStream_t stream) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (G == 64)
    hipLaunchKernelGGL(gemm_tile_kernel<64>, grid, dim3(kBlock), 0, stream, x, packed, scales, M,
                       N, K, y, d_status);
  else
    hipLaunchKernelGGL(gemm_tile_kernel<128>, grid, dim3(kBlock), 0, stream, x, packed, scales,
                       M, N, K, y, d_status);
}

}  // namespace tq
