// tq_gemv.hip -- decode GEMV / skinny matmul (1 <= M <= 16) for gfx950.
//
// y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
// (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation":
// the group scale multiplies the group's inner sum; fp32 accumulation).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// One wave per output row; lanes stride over the row's groups.
template <int G, int MT>
__global__ __launch_bounds__(kBlock) void gemv_rowwave_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scales, int M, int64_t N, int64_t K, float *__restrict__ y,
    int32_t *__restrict__ d_status) {
  constexpr int B = bytes_per_group(G);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nG = K / G;
  int flags = 0;
  for (int64_t row = (int64_t)blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave; row < N;
       row += (int64_t)gridDim.x * (kBlock / kWave)) {
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    for (int64_t g = lane; g < nG; g += kWave) {
      const float s = __half2float(__ushort_as_half(scales[row * nG + g]));
      const uint8_t *pg = packed + (row * nG + g) * B;
      const uint16_t *xg = x + g * G;
      float part[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) part[m] = 0.f;
      for (int b = 0; b < B; ++b) {
        uint32_t v = pg[b];
        if (v >= 243u) { flags |= kDevInvalidByte; continue; }
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          const uint32_t d = v % 3u;
          v /= 3u;
          const int pos = 5 * b + i;
          if (pos < G && d != 1u) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              if (m < M) {
                const float xv = bf16_to_f32(xg[(int64_t)m * K + pos]);
                part[m] += (d == 2u) ? xv : -xv;
              }
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = fmaf(s, part[m], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[m];
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
      acc[m] = v;
    }
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M) y[(int64_t)m * N + row] = acc[m];
    }
  }
  if (flags && d_status) atomicOr(d_status, flags);
}

template <int G>
void launch_g(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t M,
              int64_t N, int64_t K, float *y, int32_t *d_status, hipStream_t stream) {
  int64_t blocks = (N + 3) / 4;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  const int m = (int)M;
#define TQ_GEMV_CASE(MT)                                                                     \
  hipLaunchKernelGGL((gemv_rowwave_kernel<G, MT>), dim3(grid), dim3(kBlock), 0, stream, x, \
                     packed, scales, m, N, K, y, d_status)
  if (m <= 1) TQ_GEMV_CASE(1);
  else if (m <= 2) TQ_GEMV_CASE(2);
  else if (m <= 4) TQ_GEMV_CASE(4);
  else if (m <= 8) TQ_GEMV_CASE(8);
  else TQ_GEMV_CASE(16);
#undef TQ_GEMV_CASE
}

}  // namespace

void launch_gemv(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t M,
                 int64_t N, int64_t K, int G, float *y, int32_t *d_status, hipStream_t stream) {
  if (G == 64) launch_g<64>(x, packed, scales, M, N, K, y, d_status, stream);
  else launch_g<128>(x, packed, scales, M, N, K, y, d_status, stream);
}

}  // namespace tq
