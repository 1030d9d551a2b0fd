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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const volatile u32x4 lds_u32x4_cv;
typedef __attribute__((address_space(3))) const unsigned char lds_bytes_c;

// Core clock cycles (s_memtime) and 10 ns ticks (s_memrealtime) between two
// points of block 0's first thread, for the caller's clock estimate.
struct ClockMark {
  unsigned long long c, r;
};
__device__ __forceinline__ ClockMark clock_mark() {
  return ClockMark{__builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime()};
}
__device__ __forceinline__ void clock_store(const ClockMark &a, const ClockMark &b,
                                            unsigned long long *clocks) {
  if (clocks && blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = b.c - a.c;
    clocks[1] = b.r - a.r;
  }
}

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

// A 64 KB LDS table in the decode kernels' layout (entry e of copy j at
// e * 256 + j * 16); every thread reads eight entries per iteration, one
// 16-byte ds_read_b128 each, from copy lane % 16 at entries drawn once per
// thread.  The reads are volatile, so each iteration performs all eight.
__global__ __launch_bounds__(kThreads) void lds_table_kernel(int iters, uint32_t *__restrict__ sink,
                                                             unsigned long long *clocks) {
  __shared__ u32x4 table[4096];
  for (int i = threadIdx.x; i < 4096; i += kThreads)
    table[i] = u32x4{(uint32_t)i, (uint32_t)i * 3u, (uint32_t)i * 5u, (uint32_t)i * 7u};
  __syncthreads();
  const uint32_t copy = (threadIdx.x & 15u) * 16u;
  uint32_t st = threadIdx.x * 2654435761u + blockIdx.x * 40503u;
  uint32_t addr[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    st = st * 1664525u + 1013904223u;
    addr[u] = ((st >> 24) << 8) | copy;
  }
  lds_bytes_c *base = (lds_bytes_c *)table;
  uint32_t acc = 0;
  const ClockMark t0 = clock_mark();
  for (int it = 0; it < iters; ++it) {
    u32x4 e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) e[u] = *(lds_u32x4_cv *)(base + addr[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= e[u].x;
    // the other dwords stay live until here, so no read waits on another
#pragma unroll
    for (int u = 0; u < 8; ++u) asm volatile("" ::"v"(e[u].y), "v"(e[u].z), "v"(e[u].w));
  }
  const ClockMark t1 = clock_mark();
  clock_store(t0, t1, clocks);
  if (acc == kNever) sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Eight independent chains of one VALU instruction kind, 16 steps per
// iteration: kind 0 v_dot2_f32_bf16 (fp32 accumulate), kind 1 v_perm_b32.
template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_kernel(int iters, uint32_t *__restrict__ sink,
                                                        unsigned long long *clocks) {
  uint32_t a[8];
  float f[8];
  const uint32_t b = threadIdx.x * 0x9E3779B9u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = threadIdx.x + (uint32_t)i;
    f[i] = (float)i;
  }
  const ClockMark t0 = clock_mark();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (KIND == 0)
          f[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a[i]),
                                                 __builtin_bit_cast(bf16x2, b), f[i], false);
        else
          a[i] = __builtin_amdgcn_perm(a[i], b, 0x05040100u + (uint32_t)u);
      }
    }
  }
  const ClockMark t1 = clock_mark();
  clock_store(t0, t1, clocks);
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) x ^= a[i] ^ __float_as_uint(f[i]);
  if (x == kNever) sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = x;
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

int tq_probe_lds_table(int iters, int grid, uint32_t *sink, unsigned long long *clocks,
                       void *stream) {
  if (!sink) return TQ_ERR_NULL;
  if (iters < 1 || iters > (1 << 24) || grid < 1 || grid > 65535) return TQ_ERR_SHAPE;
  (void)hipGetLastError();
  hipLaunchKernelGGL(lds_table_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, iters, sink, clocks);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_probe_valu(int kind, int iters, int grid, uint32_t *sink, unsigned long long *clocks,
                  void *stream) {
  if (!sink) return TQ_ERR_NULL;
  if (kind < 0 || kind > 1 || iters < 1 || iters > (1 << 24) || grid < 1 || grid > 65535)
    return TQ_ERR_SHAPE;
  (void)hipGetLastError();
  if (kind == 0)
    hipLaunchKernelGGL(valu_kernel<0>, dim3((unsigned)grid), dim3(kThreads), 0,
                       (hipStream_t)stream, iters, sink, clocks);
  else
    hipLaunchKernelGGL(valu_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0,
                       (hipStream_t)stream, iters, sink, clocks);
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
