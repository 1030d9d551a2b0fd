// tq_twobit.hip -- the 2-bit ternary format on gfx950: codes from packed
// bytes, and the M = 1 decode GEMV.
//
// Format: ternary codes in two bits each, four a byte (Avenue README, size
// note: model sizes counted for 2-bit packing; "Autoregressive Language
// Model on the 6502 Processor": ternary parameters packed four a byte).
// Field f = c + 1 in {0, 1, 2}, the first weight in the lowest two bits,
// G/4 bytes a group, fp16 group scales; f = 3 is invalid.  The matmul is
// y[n] = sum_g s[n,g] sum_{j<G} x[gG+j] c[n,gG+j] (tiny-llm "Week 2 Day 3:
// Quantize the Model", "Mathematical Formulation").
//
// The GEMV: a row's bytes are cut into 16-byte chunks (64 codes: one G=64
// group or half a G=128 group, so one scale), read with aligned 16-byte
// loads.  A lane keeps one chunk position for all the rows it visits, so
// its 64 activations stay in registers as bf16 pairs; Lp lanes (16, 32 or
// 64) share a row.  A byte is one 8-byte lookup in a 256-entry LDS table of
// two bf16 code pairs (copy lane % 32, so 32 lanes never share a bank),
// multiplied in by two v_dot2_f32_bf16.  A field of 3 counts as code 0 and
// is flagged by a bitwise test on the loaded words.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kBlock = 512;
constexpr int kWaves = kBlock / 64;
constexpr int kCopies = 32;
constexpr int kRing = 4;                  // row steps in flight per lane
constexpr int kFlush = 16;                // rounds of results held in LDS per wave
constexpr int kResCap = kFlush * kRing * 4;  // floats a wave (at most 4 rows a step)
constexpr uint32_t kOOR = 0x80000000u;   // a buffer offset past any range: loads give 0
// Cache policy of the loads of packed weights and their group parameters:
// nontemporal (gfx950's nt bit), since every byte is read once.
constexpr int kStreamed = 2;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2_c;
typedef __attribute__((address_space(3))) const unsigned char lds_bytes_c;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// v from another lane of the same 16-lane DPP row (CTRL: a DPP control)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                           0xF, 0xF, false));
}

constexpr int kGemv2MaxBatch = 128;  // problems a launch (5.5 KB of kernel arguments)

// Problems of one launch: pointers, shapes, and the blocks each one takes
// (blockIdx.x past a problem's count exits at once).
struct Gemv2Batch {
  const uint16_t *x[kGemv2MaxBatch];
  const uint8_t *packed[kGemv2MaxBatch];
  const uint16_t *scales[kGemv2MaxBatch];
  float *y[kGemv2MaxBatch];
  int n[kGemv2MaxBatch], k[kGemv2MaxBatch], nblk[kGemv2MaxBatch];
};

// bf16 bits of field f's code (f = 3, invalid: 0)
__device__ __forceinline__ uint32_t code_bf16(uint32_t f) {
  return f == 0u ? 0xBF80u : (f == 2u ? 0x3F80u : 0u);
}

template <int G>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemv2_kernel(const Gemv2Batch args,
                                                       int32_t *__restrict__ d_status) {
  constexpr int CPG = G / 64;  // chunks per group
  __shared__ __align__(16) uint32_t lut[256 * kCopies * 2];
  __shared__ float res[kWaves][kResCap];
  const int p = blockIdx.y;
  const int nblk = args.nblk[p];
  if ((int)blockIdx.x >= nblk) return;  // the grid is as wide as the widest problem
  const int N = args.n[p], K = args.k[p];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // table: entry of byte b, copy c at dwords (b * kCopies + c) * 2; a thread
  // writes two copies with one 16-byte store, consecutive threads
  // consecutive copies
  for (int i = tid; i < 256 * kCopies / 2; i += kBlock) {
    const uint32_t b = (uint32_t)i / (kCopies / 2);
    const uint32_t lo = code_bf16(b & 3u) | (code_bf16((b >> 2) & 3u) << 16);
    const uint32_t hi = code_bf16((b >> 4) & 3u) | (code_bf16((b >> 6) & 3u) << 16);
    *reinterpret_cast<u32x4 *>(&lut[4 * i]) =
        u32x4{lo, hi, lo, hi};
  }

  const int L = K >> 6, nG = K / G;
  const int Lp = L <= 16 ? 16 : (L <= 32 ? 32 : 64);   // lanes a row
  const int R = 64 / Lp;                               // rows a wave step
  const int lr = lane & (Lp - 1), rs = lane / Lp;
  const bool lane_on = lr < L;

  // this lane's 64 activations, as bf16 pairs
  uint32_t xa[32];
  {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x[p], (uint32_t)K * 2u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, lane_on ? 128u * lr + 16u * i : kOOR,
                                                       0, 0));
      xa[4 * i] = v[0]; xa[4 * i + 1] = v[1]; xa[4 * i + 2] = v[2]; xa[4 * i + 3] = v[3];
    }
  }
  const uint32_t rb = (uint32_t)K / 4u;  // bytes a row
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(args.packed[p], (uint32_t)N * rb);
  const uintptr_t sp = (uintptr_t)args.scales[p];
  const uint32_t shead = (uint32_t)(sp & 3u);
  const __amdgpu_buffer_rsrc_t rs_ =
      make_rsrc((const void *)(sp - shead), ((uint32_t)N * (uint32_t)nG * 2u + shead + 3u) & ~3u);
  float *__restrict__ yp = args.y[p];
  const uint32_t copyoff = (uint32_t)(lane & (kCopies - 1)) * 8u;
  lds_bytes_c *lut_b = (lds_bytes_c *)lut;
  __syncthreads();

  // rows of this wave: first = (block * kWaves + wave) * R + rs, step RS.
  // Lanes run whole rounds of kRing steps; a step past the wave's rows loads
  // row N - 1 (kept in range) and its result is not stored.
  const int RS = nblk * kWaves * R;
  const int first = (blockIdx.x * kWaves + wv) * R;
  const int nsteps = first < N ? (N - first + RS - 1) / RS : 0;
  const int nround = (nsteps + kRing - 1) / kRing;
  u32x4 ring[kRing];
  uint32_t rsc[kRing];
  auto issue = [&](int d, int step) {
    const int r = first + rs + step * RS;
    const uint32_t row = (uint32_t)(r < N ? r : N - 1);
    ring[d] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, lane_on ? row * rb + 16u * lr : kOOR, 0,
                                                     kStreamed));
    const uint32_t so = 2u * (row * (uint32_t)nG + (uint32_t)(lr / CPG)) + shead;
    rsc[d] = __builtin_amdgcn_raw_buffer_load_b32(rs_, lane_on ? (so & ~3u) : kOOR, 0, kStreamed);
  };
#pragma unroll
  for (int d = 0; d < kRing; ++d) issue(d, d);
  uint32_t bad = 0;
  const int l16 = lane & 15;
  const bool hi8 = (l16 & 8) != 0, hi4 = (l16 & 4) != 0;
  // Results go to LDS and out to y every kFlush rounds: a global store pending
  // in the loop would make the next wait on the ring's loads a full drain
  // (stores and loads share one counter, which then no longer counts in
  // order).  A flush ends with an explicit drain, so the loop itself never
  // has a store in flight.
  int base_round = 0;  // first round whose results res holds
  auto flush = [&](int nr) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < nr * kRing * R; i += 64) {
      const int j = base_round * kRing + i / R;  // step
      const int r = first + i % R + j * RS;
      if (j < nsteps && r < N) yp[r] = res[wv][i];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __builtin_amdgcn_wave_barrier();
  };
  auto round = [&](int rnd) {
    const int s0 = rnd * kRing;
    float v[kRing];
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      const int r = first + rs + (s0 + d) * RS;
      const uint32_t row = (uint32_t)(r < N ? r : N - 1);
      const uint32_t so = 2u * (row * (uint32_t)nG + (uint32_t)(lr / CPG)) + shead;
      const float sc =
          __half2float(__ushort_as_half((unsigned short)(rsc[d] >> ((so & 2u) << 3))));
      // everything taken from the slot before it is refilled: the table
      // addresses of its 16 bytes (byte * 256 + copy offset) and the test
      // for a field of 3
      const u32x4 w = ring[d];
      uint32_t addr[16];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        addr[q] = __builtin_amdgcn_perm(copyoff, w[q >> 2], 0x0C0C0004u | ((uint32_t)(q & 3) << 8));
      bad |= ((w[0] & (w[0] >> 1)) | (w[1] & (w[1] >> 1)) | (w[2] & (w[2] >> 1)) |
              (w[3] & (w[3] >> 1))) & 0x55555555u;
      // Pin both here: computed after the refill they would keep the slot's
      // old words live beside the new load, and the register copies that
      // follow wait for that load.
      asm volatile("" : "+v"(bad));
#pragma unroll
      for (int q = 0; q < 16; ++q) asm volatile("" : "+v"(addr[q]));
      issue(d, s0 + d + kRing);  // refill the slot with the step kRing ahead
      u32x2 e[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) e[q] = *(lds_u32x2_c *)(lut_b + addr[q]);
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        acc = dot2(e[q][0], xa[2 * q], acc);
        acc = dot2(e[q][1], xa[2 * q + 1], acc);
      }
      v[d] = sc * acc;
    }
    // Sum each step's chunk values over the 16 lanes of a DPP row, four steps
    // at once: exchange across lane bit 3 (row_ror:8), then across bit 2
    // (row_half_mirror), then add within quads.  Quad k of the DPP row then
    // holds step k's sum in all four lanes.
    const float keep0 = hi8 ? v[2] : v[0], send0 = hi8 ? v[0] : v[2];
    const float keep1 = hi8 ? v[3] : v[1], send1 = hi8 ? v[1] : v[3];
    const float u0 = keep0 + dpp_f32<0x128>(send0);
    const float u1 = keep1 + dpp_f32<0x128>(send1);
    const float keep = hi4 ? u1 : u0, send = hi4 ? u0 : u1;
    float t = keep + dpp_f32<0x141>(send);
    t += dpp_f32<0xB1>(t);
    t += dpp_f32<0x4E>(t);
    // a row of Lp = 32 or 64 lanes adds its DPP rows
    if (Lp >= 32) t += __shfl_xor(t, 16);
    if (Lp >= 64) t += __shfl_xor(t, 32);
    // every lane of the row's quads holds the sum: all write it, to the
    // slot of (step, row of the step)
    const int k = l16 >> 2;  // this lane's step in the round
    res[wv][((rnd - base_round) * kRing + k) * R + rs] = t;
  };
  // The first round is peeled so that the loop is entered with its loads in
  // flight in the same order as on its back edge; it runs in every wave (a
  // wave with no rows stores nothing).
  round(0);
  for (int rnd = 1; rnd < nround; ++rnd) {
    if (rnd - base_round == kFlush) {
      flush(kFlush);
      base_round = rnd;
    }
    round(rnd);
  }
  flush(nround - base_round);
  if (bad && d_status) atomicOr(d_status, kDevInvalidByte);
}

// unpack: one thread per 16 codes (one aligned dword of packed bytes)
__global__ __launch_bounds__(kBlock) void unpack2_kernel(const uint32_t *__restrict__ packed,
                                                         uint64_t total, int8_t *__restrict__ codes,
                                                         int32_t *__restrict__ d_status) {
  int flags = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x; t < total; t += stride) {
    const uint32_t w = packed[t];
    if ((w & (w >> 1)) & 0x55555555u) flags |= kDevInvalidByte;  // a field of 3
    uint32_t out[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t x = (w >> (8 * k)) & 0xFFu;            // 4 fields
      uint32_t y = (x | (x << 12)) & 0x000F000Fu;
      y = (y | (y << 6)) & 0x03030303u;                     // one field a byte
      out[k] = __builtin_amdgcn_perm(0u, 0x000100FFu, y);   // -1, 0, +1; 3 -> 0
    }
    // nontemporal: the codes are written once and not read back here
    __builtin_nontemporal_store(u32x4{out[0], out[1], out[2], out[3]},
                                reinterpret_cast<u32x4 *>(codes + 16 * t));
  }
  if (flags && d_status) atomicOr(d_status, flags);
}

}  // namespace

void launch_unpack2(const uint8_t *packed, int64_t N, int64_t K, int G, int8_t *codes,
                    int32_t *d_status, hipStream_t stream) {
  (void)G;
  const uint64_t total = (uint64_t)N * (uint64_t)K / 16;
  uint64_t blocks = (total + kBlock - 1) / kBlock;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(unpack2_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                     reinterpret_cast<const uint32_t *>(packed), total, codes, d_status);
}

bool gemv2_supported(int64_t N, int64_t K, int G) {
  return (G == 64 || G == 128) && K % 64 == 0 && K / 64 <= 64 && N >= 1 &&
         N * (K / 4) < (int64_t(1) << 31) && N < (int64_t(1) << 28);
}

namespace {

// Blocks of one problem when it holds `share` of the launch's 512 (two
// resident a CU, so the whole grid runs in one wave of blocks), but no fewer
// than two row steps a wave.
int gemv2_blocks(int64_t N, int64_t K, int share) {
  const int L = (int)(K / 64);
  const int Lp = L <= 16 ? 16 : (L <= 32 ? 32 : 64);
  const int64_t rows_per_block = kWaves * (64 / Lp);
  int64_t blocks = share;
  const int64_t most = (N + 2 * rows_per_block - 1) / (2 * rows_per_block);
  if (blocks > most) blocks = most;
  return blocks < 1 ? 1 : (int)blocks;
}

void launch_gemv2_chunk(const Gemv2Batch &a, int n, int G, int32_t *d_status,
                        hipStream_t stream) {
  int width = 1;
  for (int i = 0; i < n; ++i) width = a.nblk[i] > width ? a.nblk[i] : width;
  const dim3 grid((unsigned)width, (unsigned)n);
  if (G == 64)
    hipLaunchKernelGGL(gemv2_kernel<64>, grid, dim3(kBlock), 0, stream, a, d_status);
  else
    hipLaunchKernelGGL(gemv2_kernel<128>, grid, dim3(kBlock), 0, stream, a, d_status);
}

}  // namespace

void launch_gemv2_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                          const uint16_t *const *scales, float *const *ys, const int64_t *Ns,
                          const int64_t *Ks, int G, int32_t *d_status, hipStream_t stream) {
  for (int c0 = 0; c0 < count; c0 += kGemv2MaxBatch) {
    const int n = count - c0 < kGemv2MaxBatch ? count - c0 : kGemv2MaxBatch;
    Gemv2Batch a{};
    for (int i = 0; i < n; ++i) {
      a.x[i] = xs[c0 + i];
      a.packed[i] = packeds[c0 + i];
      a.scales[i] = scales[c0 + i];
      a.y[i] = ys[c0 + i];
      a.n[i] = (int)Ns[c0 + i];
      a.k[i] = (int)Ks[c0 + i];
      a.nblk[i] = gemv2_blocks(Ns[c0 + i], Ks[c0 + i], 512 / n > 0 ? 512 / n : 1);
    }
    launch_gemv2_chunk(a, n, G, d_status, stream);
  }
}

void launch_gemv2_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                          const uint16_t *const *scales, float *const *ys, int64_t N, int64_t K,
                          int G, int32_t *d_status, hipStream_t stream) {
  int64_t Ns[kGemv2MaxBatch], Ks[kGemv2MaxBatch];
  for (int i = 0; i < kGemv2MaxBatch; ++i) { Ns[i] = N; Ks[i] = K; }
  for (int c0 = 0; c0 < count; c0 += kGemv2MaxBatch) {
    const int n = count - c0 < kGemv2MaxBatch ? count - c0 : kGemv2MaxBatch;
    launch_gemv2_grouped(n, xs + c0, packeds + c0, scales + c0, ys + c0, Ns, Ks, G, d_status,
                         stream);
  }
}

}  // namespace tq
