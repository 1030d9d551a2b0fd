// tq_probe.hip -- ceiling probes (include/tq_probe.h): a plain HBM read
// stream and a bf16 MFMA-only loop, timed by the benchmark so that each
// hot-path kernel's rate can be set against what this GPU reaches on plain
// work as well as against the published peaks (tiny-llm "Week 2 Day 3:
// Quantize the Model", "Revisit the Decode Roofline").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"
#include "../../include/tq_probe.h"

namespace {

constexpr int kThreads = 512;
constexpr int kInFlight = 8;
constexpr uint32_t kNever = 0x9E3779B9u;  // the sink is written only for this XOR

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Chunk c (16 bytes) of the buffer is read by thread c % T of the grid's T
// threads, in round c / T; eight rounds' loads are issued before any is
// used.
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4 *__restrict__ buf,
                                                               int64_t chunks,
                                                               uint32_t *__restrict__ sink) {
  const int64_t T = (int64_t)gridDim.x * kThreads;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  int64_t c = t;
  for (; c + (kInFlight - 1) * T < chunks; c += kInFlight * T) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) v[i] = __builtin_nontemporal_load(buf + c + i * T);
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  for (; c < chunks; c += T) {
    const u32x4 v = __builtin_nontemporal_load(buf + c);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kNever) sink[t] = acc;
}

// Eight independent accumulators per wave; operands depend on the lane so
// the compiler cannot fold the products.
__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(int64_t iters,
                                                             float *__restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63u;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + (float)((lane + i) & 7) * 0.0625f);
    b[i] = (__bf16)(0.5f - (float)((lane * 3u + i) & 7) * 0.03125f);
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  // the products are positive, so the sum is never negative infinity
  if (lane == 0 && s == -__builtin_huge_valf()) {
    const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
#pragma unroll
    for (int k = 0; k < 8; ++k) sink[w * 8 + k] = acc[k][0];
  }
}

}  // namespace

extern "C" {

int tq_probe_read_stream(const void *buf, int64_t bytes, int grid, uint32_t *sink, void *stream) {
  if (!buf || !sink) return TQ_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return TQ_ERR_ALIGN;
  if (bytes <= 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 40) || grid < 1 || grid > 65535)
    return TQ_ERR_SHAPE;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, static_cast<const u32x4 *>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_probe_mfma_bf16(int64_t iters, int grid, float *sink, void *stream) {
  if (!sink) return TQ_ERR_NULL;
  if (iters < 1 || iters > (int64_t(1) << 24) || grid < 1 || grid > 65535) return TQ_ERR_SHAPE;
  (void)hipGetLastError();
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

}  // extern "C"
