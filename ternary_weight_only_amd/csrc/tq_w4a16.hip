// tq_w4a16.hip -- W4A16 decode GEMV on gfx950: group-wise affine 4-bit
// weights times one bf16 activation row.
//
// Format (tiny-llm "Week 2 Day 3: Quantize the Model", "Group-Wise Affine
// Quantization", "Reconstruct a Stored Group", "Packed Storage Layout"):
// unsigned codes q in [0, 15], eight a uint32 with the first in the lowest
// four bits; per group of G weights of a row a bf16 scale s (either sign)
// and a bf16 bias b; w_hat = q * s + b.  The product (same page,
// "Mathematical Formulation"): y[n] = sum_g (s[n,g] sum_j x_j q_j +
// b[n,g] sum_j x_j) over the group's j, accumulated in fp32 and rounded
// once to bf16 ("Computation Flow").
//
// The GEMV: lane lr of a row (Lp lanes) owns two pieces of 32 weights,
// weights 32 lr .. 32 lr + 31 and 32 (lr + Lp) .. 32 (lr + Lp) + 31 (16 bytes
// each, each inside one group for G = 64 or 128), so each of a wave's two
// 16-byte loads per row covers contiguous bytes; its 64 activations stay in
// registers as bf16 pairs and each piece's fp32 sum serves the bias term of
// every row it visits.  A byte (two codes) is one
// 4-byte lookup in a 256-entry LDS table of bf16 code pairs (64 copies,
// lane l reads copy l, so no two lanes share a bank) and one
// v_dot2_f32_bf16; the products x * q are exact in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kBlock = 512;
constexpr int kWaves = kBlock / 64;
constexpr int kCopies = 64;
constexpr int kRing = 4;                     // row steps a round (reduced together)
constexpr int kDepth = 2;                    // row steps in flight per lane (32 bytes each)
constexpr int kFlush = 16;                   // rounds of results held in LDS per wave
constexpr int kResCap = kFlush * kRing * 4;  // floats a wave (at most 4 rows a step)
constexpr uint32_t kOOR = 0x80000000u;       // a buffer offset past any range: loads give 0
// Cache policy of the code loads: nontemporal (gfx950's nt bit); each byte
// is read once and each load instruction of a wave covers whole lines.  The
// scale and bias loads keep the default policy: a row's two pieces read
// their parameters from the same line with two instructions.
constexpr int kStreamed = 2;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const uint32_t lds_u32_c;
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

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

constexpr int kW4MaxBatch = 128;  // problems a launch (6.5 KB of kernel arguments)

// Problems of one launch: pointers, shapes, and the blocks each one takes
// (blockIdx.x past a problem's count exits at once).
struct W4Batch {
  const uint16_t *x[kW4MaxBatch];
  const uint32_t *packed[kW4MaxBatch];
  const uint16_t *scales[kW4MaxBatch];
  const uint16_t *biases[kW4MaxBatch];
  uint16_t *y[kW4MaxBatch];
  int n[kW4MaxBatch], k[kW4MaxBatch], nblk[kW4MaxBatch];
};

template <int G>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void
w4a16_gemv_kernel(const W4Batch args) {
  __shared__ __align__(16) uint32_t lut[256 * kCopies];
  __shared__ float res[kWaves][kResCap];
  const int p = blockIdx.y;
  const int nblk = args.nblk[p];
  if ((int)blockIdx.x >= nblk) return;  // the grid is as wide as the widest problem
  const int N = args.n[p], K = args.k[p];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // table: entry of byte b, copy c at dword b * kCopies + c holds the bf16
  // pair (low nibble, high nibble); a thread writes four copies with one
  // 16-byte store, consecutive threads consecutive copies
  for (int i = tid; i < 256 * kCopies / 4; i += kBlock) {
    const uint32_t b = (uint32_t)i / (kCopies / 4);
    const uint32_t e = (__float_as_uint((float)(b & 15u)) >> 16) |
                       (__float_as_uint((float)(b >> 4)) & 0xFFFF0000u);
    *reinterpret_cast<u32x4 *>(&lut[4 * i]) = u32x4{e, e, e, e};
  }

  const int L = K >> 6, nG = K / G;
  const int Lp = L <= 16 ? 16 : (L <= 32 ? 32 : 64);  // lanes a row
  const int R = 64 / Lp;                              // rows a wave step
  const int lr = lane & (Lp - 1), rs = lane / Lp;
  // The lane's two 32-code pieces of a row: A = bytes [16 lr, 16 lr + 16), B
  // = bytes [16 (lr + Lp), ...), so each load instruction of a wave covers
  // whole lines of the row (and can use the nontemporal policy).  A piece
  // lies in one group; pieces past the row's K/2 bytes read zeros.
  const uint32_t rbytes = (uint32_t)K / 2u;
  const bool onA = 16u * (uint32_t)lr < rbytes, onB = 16u * (uint32_t)(lr + Lp) < rbytes;
  const uint32_t gA = 32u * (uint32_t)lr / (uint32_t)G, gB = 32u * (uint32_t)(lr + Lp) / (uint32_t)G;

  // this lane's 64 activations as bf16 pairs, and their sum
  uint32_t xa[32];
  float xsumA = 0.f, xsumB = 0.f;
  {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x[p], (uint32_t)K * 2u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rx, i < 4 ? (onA ? 64u * lr + 16u * i : kOOR)
                               : (onB ? 64u * (uint32_t)(lr + Lp) + 16u * (i - 4) : kOOR),
                     0, 0));
      xa[4 * i] = v[0]; xa[4 * i + 1] = v[1]; xa[4 * i + 2] = v[2]; xa[4 * i + 3] = v[3];
    }
  }
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(args.packed[p], (uint32_t)N * rbytes);
  // scales and biases: bf16, read as the dword holding the lane's one
  const uintptr_t sp = (uintptr_t)args.scales[p], bp = (uintptr_t)args.biases[p];
  const uint32_t shead = (uint32_t)(sp & 3u), bhead = (uint32_t)(bp & 3u);
  const uint32_t sbytes = (uint32_t)N * (uint32_t)nG * 2u;
  const __amdgpu_buffer_rsrc_t rsc_ =
      make_rsrc((const void *)(sp - shead), (sbytes + shead + 3u) & ~3u);
  const __amdgpu_buffer_rsrc_t rbi_ =
      make_rsrc((const void *)(bp - bhead), (sbytes + bhead + 3u) & ~3u);
  uint16_t *__restrict__ yp = args.y[p];
  const uint32_t copyoff = (uint32_t)lane * 4u;
  lds_bytes_c *lut_b = (lds_bytes_c *)lut;
  __syncthreads();

  // rows of this wave: first = (block * kWaves + wave) * R + rs, step RS.
  // Lanes run whole rounds of kRing steps; a step past the wave's rows loads
  // row N - 1 (kept in range) and its result is not stored.
  const int RS = nblk * kWaves * R;
  const int first = (blockIdx.x * kWaves + wv) * R;
  const int nsteps = first < N ? (N - first + RS - 1) / RS : 0;
  const int nround = (nsteps + kRing - 1) / kRing;
  u32x4 ring_a[kDepth], ring_b[kDepth];
  uint32_t rswA[kDepth], rbwA[kDepth], rswB[kDepth], rbwB[kDepth];
  auto param_off = [&](uint32_t row, uint32_t g, uint32_t head) {
    return 2u * (row * (uint32_t)nG + g) + head;
  };
  // a piece past the row reads past every range (offsets stay below 2^31, so
  // setting bit 31 is enough): an OR, where a select was turned into a
  // branch around each load, and a load under a branch makes the next wait
  // a full drain
  const uint32_t maskA = onA ? 0u : kOOR, maskB = onB ? 0u : kOOR;
  auto issue = [&](int d, int step) {
    const int r = first + rs + step * RS;
    const uint32_t row = (uint32_t)(r < N ? r : N - 1);
    const uint32_t o = row * rbytes + 16u * (uint32_t)lr;
    ring_a[d] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, o | maskA, 0, kStreamed));
    ring_b[d] = __builtin_bit_cast(
        u32x4,
        __builtin_amdgcn_raw_buffer_load_b128(rp, (o + 16u * (uint32_t)Lp) | maskB, 0, kStreamed));
    rswA[d] = __builtin_amdgcn_raw_buffer_load_b32(
        rsc_, (param_off(row, gA, shead) & ~3u) | maskA, 0, 0);
    rbwA[d] = __builtin_amdgcn_raw_buffer_load_b32(
        rbi_, (param_off(row, gA, bhead) & ~3u) | maskA, 0, 0);
    rswB[d] = __builtin_amdgcn_raw_buffer_load_b32(
        rsc_, (param_off(row, gB, shead) & ~3u) | maskB, 0, 0);
    rbwB[d] = __builtin_amdgcn_raw_buffer_load_b32(
        rbi_, (param_off(row, gB, bhead) & ~3u) | maskB, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(d, d);
  // the activations' sum once the ring's first loads are out
#pragma unroll
  for (int j = 0; j < 16; ++j) {  // x0 + x1 per pair, for each piece
    xsumA = dot2(xa[j], 0x3F803F80u, xsumA);
    xsumB = dot2(xa[16 + j], 0x3F803F80u, xsumB);
  }
  const int l16 = lane & 15;
  const bool hi8 = (l16 & 8) != 0, hi4 = (l16 & 4) != 0;
  // Results go to LDS and out to y every kFlush rounds: a global store
  // pending in the loop would make the next wait on the ring's loads a full
  // drain (stores and loads share one counter, which then no longer counts
  // in order).  A flush ends with an explicit drain.
  int base_round = 0;  // first round whose results res holds
  auto flush = [&](int nr) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < nr * kRing * R; i += 64) {
      const int j = base_round * kRing + i / R;  // step
      const int r = first + i % R + j * RS;
      if (j < nsteps && r < N) yp[r] = f32_to_bf16_rne(res[wv][i]);
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
      const int sl = d % kDepth;
      const float scA =
          bf16_to_f32((rswA[sl] >> ((param_off(row, gA, shead) & 2u) << 3)) & 0xFFFFu);
      const float biA =
          bf16_to_f32((rbwA[sl] >> ((param_off(row, gA, bhead) & 2u) << 3)) & 0xFFFFu);
      const float scB =
          bf16_to_f32((rswB[sl] >> ((param_off(row, gB, shead) & 2u) << 3)) & 0xFFFFu);
      const float biB =
          bf16_to_f32((rbwB[sl] >> ((param_off(row, gB, bhead) & 2u) << 3)) & 0xFFFFu);
      // the table addresses of the slot's 32 bytes (byte * 256 + copy offset),
      // pinned before the refill: computed after it they would keep the
      // slot's old words live beside the new load, and the register copies
      // that follow wait for that load
      uint32_t addr[32];
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const uint32_t w = q < 16 ? ring_a[sl][q >> 2] : ring_b[sl][(q - 16) >> 2];
        addr[q] = __builtin_amdgcn_perm(copyoff, w, 0x0C0C0004u | ((uint32_t)(q & 3) << 8));
      }
#pragma unroll
      for (int q = 0; q < 32; ++q) asm volatile("" : "+v"(addr[q]));
      issue(sl, s0 + d + kDepth);  // refill the slot with the step kDepth ahead
      float acc[2] = {0.f, 0.f};
      // the two pieces of 16 bytes, each looked up in full before its products
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t e[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) e[q] = *(lds_u32_c *)(lut_b + addr[16 * h + q]);
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[h] = dot2(e[q], xa[16 * h + q], acc[h]);
        // the products now: sunk to the round's end they would hold every
        // step's lookups at once
        asm volatile("" : "+v"(acc[h]));
      }
      v[d] = scA * acc[0] + biA * xsumA + (scB * acc[1] + biB * xsumB);
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
}

}  // namespace

bool w4a16_gemv_supported(int64_t N, int64_t K, int G) {
  return (G == 64 || G == 128) && K % 64 == 0 && K / 64 <= 64 && N >= 1 &&
         N * (K / 2) < (int64_t(1) << 31) && N < (int64_t(1) << 28);
}

namespace {

// Blocks of one problem when it holds `share` of the launch's 512 (two
// resident a CU, so the whole grid runs in one wave of blocks), but no fewer
// than two row steps a wave.
int w4_blocks(int64_t N, int64_t K, int share) {
  const int L = (int)(K / 64);
  const int Lp = L <= 16 ? 16 : (L <= 32 ? 32 : 64);
  const int64_t rows_per_block = kWaves * (64 / Lp);
  int64_t blocks = share;
  const int64_t most = (N + 2 * rows_per_block - 1) / (2 * rows_per_block);
  if (blocks > most) blocks = most;
  return blocks < 1 ? 1 : (int)blocks;
}

}  // namespace

void launch_w4a16_gemv_grouped(int count, const uint16_t *const *xs,
                               const uint32_t *const *packeds, const uint16_t *const *scales,
                               const uint16_t *const *biases, uint16_t *const *ys,
                               const int64_t *Ns, const int64_t *Ks, int G, hipStream_t stream) {
  for (int c0 = 0; c0 < count; c0 += kW4MaxBatch) {
    const int n = count - c0 < kW4MaxBatch ? count - c0 : kW4MaxBatch;
    W4Batch a{};
    int width = 1;
    for (int i = 0; i < n; ++i) {
      a.x[i] = xs[c0 + i];
      a.packed[i] = packeds[c0 + i];
      a.scales[i] = scales[c0 + i];
      a.biases[i] = biases[c0 + i];
      a.y[i] = ys[c0 + i];
      a.n[i] = (int)Ns[c0 + i];
      a.k[i] = (int)Ks[c0 + i];
      a.nblk[i] = w4_blocks(Ns[c0 + i], Ks[c0 + i], 512 / n > 0 ? 512 / n : 1);
      width = a.nblk[i] > width ? a.nblk[i] : width;
    }
    const dim3 grid((unsigned)width, (unsigned)n);
    if (G == 64)
      hipLaunchKernelGGL(w4a16_gemv_kernel<64>, grid, dim3(kBlock), 0, stream, a);
    else
      hipLaunchKernelGGL(w4a16_gemv_kernel<128>, grid, dim3(kBlock), 0, stream, a);
  }
}

void launch_w4a16_gemv_batched(int count, const uint16_t *const *xs,
                               const uint32_t *const *packeds, const uint16_t *const *scales,
                               const uint16_t *const *biases, uint16_t *const *ys, int64_t N,
                               int64_t K, int G, hipStream_t stream) {
  int64_t Ns[kW4MaxBatch], Ks[kW4MaxBatch];
  for (int i = 0; i < kW4MaxBatch; ++i) { Ns[i] = N; Ks[i] = K; }
  for (int c0 = 0; c0 < count; c0 += kW4MaxBatch) {
    const int n = count - c0 < kW4MaxBatch ? count - c0 : kW4MaxBatch;
    launch_w4a16_gemv_grouped(n, xs + c0, packeds + c0, scales + c0, biases + c0, ys + c0, Ns,
                              Ks, G, stream);
  }
}

}  // namespace tq
