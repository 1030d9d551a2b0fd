// tq_dequant.hip -- decode packed ternary codes and fp16 group scales into a
// bf16 weight matrix, w_hat[n,k] = bf16(c[n,k] * s[n,k/G]), for gfx950.
//
// Format and rule: precisit "pack-unpack-run" README, codec.py description
// (decoding gives back c * s; five base-3 digits c + 1 per byte, first
// weight least significant; each group byte-aligned with zero-trit padding;
// byte values 243..255 invalid) and screen.py description (the decoder
// hands the selected weights back as bf16).
//
// The work is a stream: per group of G weights, ceil(G/5) packed bytes and a
// 2-byte scale in, 2G bytes out, so the written bf16 matrix is ~90% of the
// traffic and the kernel is bound by HBM writes.  One thread makes 8
// consecutive weights of one group (G % 8 == 0) and writes them with one
// 16-byte store, so a wave writes 1 KB contiguously.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_digits.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kBlock = 256;
constexpr int kMaxBlocks = 65536;  // blocks of one launch, over all its problems
constexpr int kMinBlocks = 2048;   // 8 per CU: below this, fewer items per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 bits of the fp16 value h (finite): fp16 -> fp32 is exact, then one
// round to nearest, ties to even, to 8 significant bits.  Every finite fp16
// lies inside bf16's normal range, so nothing overflows or goes subnormal.
__device__ __forceinline__ uint32_t bf16_of_f16(uint32_t h) {
  const float f = __half2float(__ushort_as_half((unsigned short)h));
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Problems of one launch: blockIdx.y picks the problem, all of one shape.
struct DequantBatch {
  const uint8_t *packed[kDequantMaxBatch];
  const uint16_t *scales[kDequantMaxBatch];
  uint16_t *w_hat[kDequantMaxBatch];
};

// U items of 8 weights per thread and pass, all of their loads issued
// before any of them is decoded.
template <int G, int U>
__global__ __launch_bounds__(kBlock) void dequant_kernel(const DequantBatch args, uint64_t total,
                                                         int32_t *__restrict__ d_status) {
  const uint8_t *__restrict__ packed = args.packed[blockIdx.y];
  const uint16_t *__restrict__ scales = args.scales[blockIdx.y];
  uint16_t *__restrict__ w_hat = args.w_hat[blockIdx.y];
  constexpr int TPG = G / 8;              // threads per group
  constexpr int B = bytes_per_group(G);
  constexpr int NPAD = 5 * B - G;         // padding trits, all in the group's last byte
  constexpr uint32_t kPadMask = (1u << (2 * NPAD)) - 1u;
  constexpr uint32_t kPadZero = 0x5555u & kPadMask;  // digits 1 = code 0

  __shared__ uint32_t lut[256];
  lut[threadIdx.x] = digit_entry(threadIdx.x);
  __syncthreads();

  // Packed bytes are read as aligned dwords counted from the dword holding
  // packed[0]; a dword read always holds a byte of the thread's own group,
  // so no read leaves the buffer's pages.
  const uint32_t pmis = (uint32_t)(reinterpret_cast<uintptr_t>(packed) & 3u);
  const uint32_t *__restrict__ pw = reinterpret_cast<const uint32_t *>(packed - pmis);

  int flags = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  // U items per thread and pass, all loads issued before any is used.
  for (uint64_t t0 = (uint64_t)blockIdx.x * kBlock + threadIdx.x; t0 < total; t0 += U * stride) {
    uint32_t w0[U], w1[U], h[U], sh[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint64_t t = t0 + u * stride;
      t = t < total ? t : total - 1;       // past the end: reload the last item, store nothing
      const uint64_t gi = t / TPG;
      const int p0 = (int)(t % TPG) * 8;
      const int b0 = p0 / 5, o = p0 - 5 * b0;
      const int nb = (o + 12) / 5;         // bytes holding weights p0..p0+7: 2 or 3
      const uint64_t r = gi * B + b0 + pmis;
      w0[u] = pw[r >> 2];
      w1[u] = pw[(r + nb - 1) >> 2];
      sh[u] = 8u * (uint32_t)(r & 3u);
      h[u] = scales[gi];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t t = t0 + u * stride;
      if (t >= total) break;
      const uint64_t gi = t / TPG;
      const int p0 = (int)(t % TPG) * 8;   // first weight of this item in its group
      const int b0 = p0 / 5, o = p0 - 5 * b0;
      const int nb = (o + 12) / 5;
      const uint32_t bytes = (uint32_t)((((uint64_t)w1[u] << 32) | w0[u]) >> sh[u]);

      const uint32_t e0 = lut[bytes & 0xFFu];
      const uint32_t e1 = lut[(bytes >> 8) & 0xFFu];
      const uint32_t e2 = nb == 3 ? lut[(bytes >> 16) & 0xFFu] : 0u;
      if ((e0 | e1 | e2) & kLutInvalid) flags |= kDevInvalidByte;
      // digits of weights p0 .. p0+7 in bits 0..15, then the next ones
      const uint32_t d =
          ((e0 & 0x3FFu) | ((e1 & 0x3FFu) << 10) | ((e2 & 0x3FFu) << 20)) >> (2 * o);
      if (p0 + 8 == G && ((d >> 16) & kPadMask) != kPadZero) flags |= kDevBadPadding;

      // The three values a weight can take: c = -1, 0, +1 times s, each the
      // IEEE product (a zero carries the sign of c * s).  A non-finite scale
      // gives a zero group.
      const bool finite = ((h[u] >> 10) & 0x1Fu) != 0x1Fu;
      if (!finite) flags |= kDevNonfinite;
      const uint32_t sb = finite ? bf16_of_f16(h[u]) : 0u;
      const uint32_t lo = finite ? ((sb ^ 0x8000u) | ((sb & 0x8000u) << 16)) : 0u;  // -s | +-0
      const uint32_t hi = sb | (sb << 16);                                          // +s | +s

      // Pair k of weights takes bytes 2d, 2d+1 of {hi, lo} for each digit d
      // (0..1 is -s, 2..3 the zero, 4..5 +s).
      uint32_t out[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t dd = (d >> (4 * k)) & 0xFu;
        const uint32_t pair = (dd & 3u) | ((dd >> 2) << 16);
        out[k] = __builtin_amdgcn_perm(hi, lo, pair * 0x0202u + 0x01000100u);
      }
      // a non-temporal store: the output is not read back by this kernel
      const u32x4 v = {out[0], out[1], out[2], out[3]};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(w_hat + gi * G + p0));
    }
  }
  if (flags && d_status) atomicOr(d_status, flags);
}

}  // namespace

template <int G, int U>
void launch_u(const DequantBatch &a, int n, uint64_t total, int32_t *d_status,
              hipStream_t stream) {
  // one pass of U items per thread, or, past kMaxBlocks in the launch, fewer
  // blocks that stride; every problem gets the same number of blocks
  uint64_t blocks = (total + kBlock * U - 1) / (kBlock * U);
  const uint64_t cap = (uint64_t)(kMaxBlocks / n);
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((dequant_kernel<G, U>), dim3((unsigned)blocks, (unsigned)n), dim3(kBlock),
                     0, stream, a, total, d_status);
}

template <int G>
void launch_g(const DequantBatch &a, int n, uint64_t total, int32_t *d_status,
              hipStream_t stream) {
  // the most items per thread that still leaves kMinBlocks blocks
  const uint64_t b4 = (total + kBlock * 4 - 1) / (kBlock * 4) * (uint64_t)n;
  if (b4 >= (uint64_t)kMinBlocks)
    launch_u<G, 4>(a, n, total, d_status, stream);
  else if (2 * b4 >= (uint64_t)kMinBlocks)
    launch_u<G, 2>(a, n, total, d_status, stream);
  else
    launch_u<G, 1>(a, n, total, d_status, stream);
}

void launch_dequantize_batched(int count, const uint8_t *const *packeds,
                               const uint16_t *const *scales, uint16_t *const *w_hats, int64_t N,
                               int64_t K, int G, int32_t *d_status, hipStream_t stream) {
  const uint64_t total = (uint64_t)N * (uint64_t)K / 8;  // items of 8 weights per problem
  for (int c0 = 0; c0 < count; c0 += kDequantMaxBatch) {
    const int n = count - c0 < kDequantMaxBatch ? count - c0 : kDequantMaxBatch;
    DequantBatch a{};
    for (int i = 0; i < n; ++i) {
      a.packed[i] = packeds[c0 + i];
      a.scales[i] = scales[c0 + i];
      a.w_hat[i] = w_hats[c0 + i];
    }
    if (G == 64)
      launch_g<64>(a, n, total, d_status, stream);
    else
      launch_g<128>(a, n, total, d_status, stream);
  }
}

void launch_dequantize(const uint8_t *packed, const uint16_t *scales, int64_t N, int64_t K, int G,
                       uint16_t *w_hat, int32_t *d_status, hipStream_t stream) {
  launch_dequantize_batched(1, &packed, &scales, &w_hat, N, K, G, d_status, stream);
}

}  // namespace tq
