// tq_gemm.hip -- prefill matmul for gfx950.
//
// y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
// (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation";
// prefill reuses each weight tile across many rows, "Revisit the Decode
// Roofline").
//
// Schedule:
//   * A block of 4 waves computes a 128 x 128 tile of y; each wave owns a
//     64 x 64 sub-tile of 16x16 MFMA tiles (v_mfma_f32_16x16x32_bf16: bf16
//     inputs, fp32 accumulation).  A block takes 80 KiB of LDS, so two blocks
//     share a CU and fill each other's barrier and latency gaps.
//   * K is walked in stages of 32.  Per stage s:
//       - the activations of stage s+3 go from memory straight into their
//         slot of a 4-slot LDS ring (buffer loads with the lds modifier: no
//         registers; lane l of a wave lands 16 l bytes past the wave's base);
//       - the packed bytes of stage s+1, loaded two stages earlier into a
//         register ring, are looked up in the decode table, and the bytes of
//         stage s+3 are requested;
//       - the stage's 16 MFMAs per wave run, and the codes of stage s+1 are
//         assembled and written to the other of two code slots;
//       - one barrier, after a wait that leaves the younger loads in flight.
//   * Codes enter the MFMA as the bf16 value 2c in {-2, 0, 2}: exact, and its
//     low byte is zero, so a pair of codes is one v_perm of table bytes.  At
//     the end of a group its fp32 partial is scaled by s/2 (exact) and added
//     to the fp32 accumulator, so the fp16 scale is never rounded.
//   * The decode table maps a byte to the high bytes of its five codes (8
//     bytes per entry, 16 copies so that a 16-lane phase of random lookups
//     hits distinct banks).  Entries 243..255 carry a flag byte that is OR-ed
//     up and reported as TQ_DEV_INVALID_BYTE.
//   * Tiles are stored without padding; the 16-byte chunk kc of row r sits at
//     chunk kc ^ ((r >> 1) & 3) of its 64-byte row, which keeps the operand
//     reads and the code writes free of bank conflicts.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_bytes;
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2_c;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_c;

constexpr int kWave = 64;
constexpr int BM = 128;                 // activation rows per block
constexpr int BN = 128;                 // weight rows per block
constexpr int NT = 256;                 // threads per block
constexpr int KS = 32;                  // K values per stage
constexpr int XRING = 4;                // activation slots
constexpr int XSLOT = BM * KS * 2;      // 8 KiB
constexpr int CSLOT = BN * KS * 2;      // 8 KiB
constexpr int kCopies = 16;
constexpr int kEntryBytes = 8;
constexpr int LUTB = 256 * kCopies * kEntryBytes;  // 32 KiB
constexpr uint32_t kCsOff = XRING * XSLOT;
constexpr uint32_t kLutOff = kCsOff + 2 * CSLOT;
constexpr int SMEM = kLutOff + LUTB;    // 80 KiB
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr uint32_t kBadFlag = 0xFF00u;  // in the high dword of entries 243..255

struct GemmBatch {
  const uint16_t *x[kGemmMaxBatch];
  const uint8_t *packed[kGemmMaxBatch];
  const uint16_t *scales[kGemmMaxBatch];
  float *y[kGemmMaxBatch];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// byte offset of 16-byte chunk kc (0..3) of row r in a swizzled tile; this
// placement was measured bank-conflict free on gfx950 both for the operand
// reads (16 rows x 4 chunks per instruction) and for the code writes (64
// rows x one chunk), where the padded and the (r >> 2) layouts conflict 2-way
__device__ __forceinline__ uint32_t swz(uint32_t r, uint32_t kc) {
  return 16u * (4u * r + (kc ^ ((r >> 1) & 3u)));
}

// Table entry for byte e: high bytes of 2*c_i (0xC0 for -2, 0x00, 0x40 for
// +2), i = 0..3 in the low dword, i = 4 in byte 0 of the high dword.
__device__ __forceinline__ u32x2 code_entry(uint32_t e) {
  if (e >= 243u) return u32x2{0u, kBadFlag};
  uint32_t h[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t d = e % 3u;
    e /= 3u;
    h[i] = d == 0u ? 0xC0u : (d == 2u ? 0x40u : 0u);
  }
  return u32x2{h[0] | (h[1] << 8) | (h[2] << 16) | (h[3] << 24), h[4]};
}

// A run of 16 codes starts at digit D0 of its first byte; lo/hi are the table
// entries of the run's four bytes.  Output dword w is the bf16 pair
// (2c_{2w}, 2c_{2w+1}) of the run.
template <int D0>
__device__ __forceinline__ void stitch(const uint32_t (&lo)[4], const uint32_t (&hi)[4],
                                       uint32_t (&out)[8]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int h1 = D0 + 2 * w, j1 = h1 / 5, o1 = h1 % 5;
    const int h2 = h1 + 1, j2 = h2 / 5, o2 = h2 % 5;
    // v_perm byte pool: src1 = bytes 0..3, src0 = bytes 4..7; selector 0x0C
    // gives a zero byte
    uint32_t s0, s1;
    int b1, b2;
    if (j1 == j2 && o2 <= 3) {
      s0 = lo[j1]; s1 = lo[j1]; b1 = o1; b2 = o2;
    } else if (j1 == j2) {  // digits 3 and 4 of one byte
      s0 = hi[j1]; s1 = lo[j1]; b1 = 3; b2 = 4;
    } else {                // digit 4 of byte j1, digit 0 of byte j2
      s0 = hi[j1]; s1 = lo[j2]; b1 = 4; b2 = 0;
    }
    out[w] = __builtin_amdgcn_perm(s0, s1, 0x000C000Cu | ((uint32_t)b1 << 8) | ((uint32_t)b2 << 24));
  }
}

template <int V>
struct Int {
  static constexpr int value = V;
};

template <int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_kernel(const GemmBatch args, int M, int N, int K, int64_t ldy,
                 int32_t *__restrict__ d_status) {
  constexpr int B = bytes_per_group(G);  // 13 or 26
  constexpr int SPG = G / KS;            // stages per group: 2 or 4
  constexpr int TM = 4;                  // 16-row MFMA tiles per wave (and TN = 4 columns)

  __shared__ __align__(16) unsigned char smem_raw[SMEM];
  lds_bytes *smem = (lds_bytes *)smem_raw;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int wm = wv >> 1, wn = wv & 1;
  const int tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
  const int tpp = tilesM * tilesN;
  const int pi = (int)blockIdx.x / tpp;
  const int t = (int)blockIdx.x - pi * tpp;
  const int m0 = (t % tilesM) * BM, n0 = (t / tilesM) * BN;
  const int nG = K / G, nS = K / KS;
  const uint32_t rowbytes = (uint32_t)nG * B;
  const int mrows = min(BM, M - m0), nrows = min(BN, N - n0);

  // Buffer descriptors based at this block's tiles: 32-bit offsets suffice.
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(args.x[pi] + (int64_t)m0 * K, (uint32_t)mrows * (uint32_t)K * 2u);
  const uintptr_t pabs = reinterpret_cast<uintptr_t>(args.packed[pi]) + (uint64_t)n0 * rowbytes;
  const uint32_t pbase = (uint32_t)(pabs & 3u);  // packed has any alignment
  // The range is a whole number of dwords, so a dword load is either fully
  // in range or fully past it (then it reads 0).
  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(reinterpret_cast<const void *>(pabs - pbase),
                (pbase + (uint32_t)nrows * rowbytes + 3u) & ~3u);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(args.scales[pi] + (int64_t)n0 * nG, (uint32_t)nrows * (uint32_t)nG * 2u);

  // ---- decode table: thread e writes the 16 copies of entry e, the copy
  // index rotated by e to spread the banks ----
  {
    const u32x2 v = code_entry((uint32_t)tid);
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      const uint32_t j = (uint32_t)((k + tid) & (kCopies - 1));
      *(lds_u32x2 *)(smem + kLutOff + ((uint32_t)tid * kCopies + j) * kEntryBytes) = v;
    }
  }

  // Every stage issues the same loads -- past the end they read junk or
  // zeros into slots that are never consumed -- so the wait counts are fixed.
  const uint32_t wvs = __builtin_amdgcn_readfirstlane(wv);  // wave index, scalar
  // ---- activations: op i of thread t fills chunk 256 i + t of the slot.
  // Offsets stay in the per-lane offset, the only part of a raw buffer
  // address that is range-checked (the scalar offset is not). ----
  uint32_t xoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t U = 256u * i + (uint32_t)tid;
    const uint32_t r = U >> 2, kc = (U & 3u) ^ ((r >> 1) & 3u);  // inverse of swz
    xoff[i] = (int)r < mrows ? ((uint32_t)r * (uint32_t)K + kc * 8u) * 2u : kOutOfRange;
  }
  auto dma_x = [&](int s) {
    const uint32_t slot = (uint32_t)(s & (XRING - 1)) * XSLOT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lds_bytes *dst = smem + slot + 16u * (256u * i + 64u * wvs);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void *)dst,
                                               16, xoff[i] + (uint32_t)s * (KS * 2), 0, 0, 0);
    }
  };

  // ---- scales: lanes hold column n = wn*64 + tn*16 + (lane & 15) ----
  constexpr int TN = 4;
  uint32_t soff[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int n = wn * 64 + tn * 16 + (lane & 15);
    soff[tn] = n < nrows ? 2u * (uint32_t)n * (uint32_t)nG : kOutOfRange;
  }
  uint32_t sc_cur[TN], sc_next[TN];
  auto load_scales = [&](int g, uint32_t (&dst)[TN]) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      dst[tn] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[tn] + 2u * (uint32_t)g, 0, 0);
  };

  // ---- packed bytes: thread (row dr, half dq) decodes codes 16 dq .. 16 dq
  // + 15 of each stage; two dwords hold the run's four bytes ----
  const int dr = tid & (BN - 1);
  const uint32_t dqs = __builtin_amdgcn_readfirstlane(tid >> 7);  // uniform over a wave
  const bool drow_on = dr < nrows;
  const uint32_t prow = drow_on ? pbase + (uint32_t)dr * rowbytes : kOutOfRange;
  const uint32_t lut_lane = kLutOff + (uint32_t)(tid & (kCopies - 1)) * kEntryBytes;
  uint32_t flags = 0;
  auto lookup = [&](const uint32_t (&raw)[2], uint32_t ofs, uint32_t (&lo)[4], uint32_t (&hi)[4]) {
    const uint32_t w = __builtin_amdgcn_alignbyte(raw[1], raw[0], ofs);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t b = (w >> (8 * k)) & 0xFFu;
      const u32x2 e = *(lds_u32x2_c *)(smem + ((b << 7) + lut_lane));
      lo[k] = e.x;
      hi[k] = e.y;
    }
  };

  // ---- MFMA operands: lane reads rows r0 + 16 a, chunk lane >> 4 ----
  const uint32_t kq = (uint32_t)(lane >> 4);
  const uint32_t aoff = swz((uint32_t)(wm * 64 + (lane & 15)), kq);
  const uint32_t boff = kCsOff + swz((uint32_t)(wn * 64 + (lane & 15)), kq);

  f32x4 acc[TM][TN], part[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      part[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // The rest is instantiated per decode half DQ (uniform over a wave), so
  // that each stage is one branch-free block the scheduler can interleave.
  auto body = [&](auto dqc) {
    constexpr int DQ = decltype(dqc)::value;
    auto load_packed = [&](int s, uint32_t (&dst)[2], uint32_t &ofs) {
      const int g = s / SPG, st = s % SPG;
      const uint32_t a = prow + (uint32_t)(g * B + (st * KS + 16 * DQ) / 5);
      ofs = a & 3u;
      const uint32_t a4 = a & ~3u;
      dst[0] = __builtin_amdgcn_raw_buffer_load_b32(rp, a4, 0, 0);
      dst[1] = __builtin_amdgcn_raw_buffer_load_b32(rp, a4 + 4u, 0, 0);
    };
    // codes of a run that is stage ST of its group -> two chunks of slot cs
    auto emit = [&](auto stc, const uint32_t (&lo)[4], const uint32_t (&hi)[4], uint32_t cs) {
      constexpr int ST = decltype(stc)::value;
      flags |= (hi[0] | hi[1]) | (hi[2] | hi[3]);
      uint32_t out[8];
      stitch<(ST * KS + 16 * DQ) % 5>(lo, hi, out);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *(lds_u32x4 *)(smem + cs + swz((uint32_t)dr, (uint32_t)(2 * DQ + i))) =
            u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
    };

    // ---- prologue: all of it completes before the loop, so the compiler's
    // wait counts inside the loop need not cover it ----
    uint32_t ring[2][2], rofs[2], first[2], first_ofs;
    load_scales(0, sc_cur);
    dma_x(0);
    dma_x(1);
    dma_x(2);
    load_packed(0, first, first_ofs);
    load_packed(1, ring[1], rofs[1]);
    load_packed(2, ring[0], rofs[0]);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    __syncthreads();                // table and stage 0 activations ready
    {
      uint32_t lo[4], hi[4];
      lookup(first, first_ofs, lo, hi);
      emit(Int<0>{}, lo, hi, kCsOff);
    }
    __syncthreads();

    // stage s is stage ST of its group; it reads code slot ST & 1
    auto stage = [&](auto stc, int s) {
      constexpr int ST = decltype(stc)::value;
      constexpr int P = ST & 1, Q = 1 - P;
      constexpr int ST1 = (ST + 1) % SPG;  // place of stage s+1 in its group
      // table lookups for stage s+1: its bytes were requested two stages ago
      // (past the last stage they decode junk into the free code slot)
      uint32_t lo[4], hi[4];
      lookup(ring[Q], rofs[Q], lo, hi);
      const uint32_t xs = (uint32_t)(s & (XRING - 1)) * XSLOT;
      bf16x8 av[TM], bv[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) av[a] = *(lds_bf16x8_c *)(smem + xs + aoff + 1024u * a);
#pragma unroll
      for (int b = 0; b < TN; ++b) bv[b] = *(lds_bf16x8_c *)(smem + P * CSLOT + boff + 1024u * b);
      if (ST == 0) load_scales(s / SPG + 1, sc_next);
      dma_x(s + 3);
      load_packed(s + 3, ring[Q], rofs[Q]);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          part[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              av[a], bv[b], ST == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : part[a][b], 0, 0, 0);
      emit(Int<ST1>{}, lo, hi, kCsOff + (uint32_t)Q * CSLOT);
      if (ST == SPG - 1) {
        // end of a group: acc += (s/2) * part (codes entered as 2c)
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const float sh = 0.5f * __half2float(__ushort_as_half((unsigned short)sc_cur[b]));
#pragma unroll
          for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[a][b][r] = fmaf(sh, part[a][b][r], acc[a][b][r]);
        }
#pragma unroll
        for (int b = 0; b < TN; ++b) sc_cur[b] = sc_next[b];
      }
      // Instruction order for the scheduler: the table and operand reads and
      // the loads first, then each MFMA followed by vector-ALU work, so that
      // the decode and the scaling run in the MFMA shadow.
      constexpr int kValu = ST == SPG - 1 ? 6 : 1;
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // VALU: table addresses
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // DS reads
      __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);   // VMEM reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);   // DS writes
      // The activations of stage s+1 (requested two stages ago) must have
      // landed before the barrier; at least ten younger loads (the
      // activations of stages s+2 and s+3, the bytes of stages s+1 .. s+3)
      // may stay in flight.
      asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    for (int s = 0; s < nS; s += SPG) {  // nS is a multiple of SPG
      stage(Int<0>{}, s);
      stage(Int<1>{}, s + 1);
      if constexpr (SPG == 4) {
        stage(Int<2>{}, s + 2);
        stage(Int<3>{}, s + 3);
      }
    }
  };
  if (dqs == 0)
    body(Int<0>{});
  else
    body(Int<1>{});
  // no load may still be writing this block's LDS when it exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane holds column (lane & 15), rows 4*(lane>>4) + r; y is
  // written with nontemporal stores (never read back here) ----
  const int mb = wm * 64 + 4 * (lane >> 4), nb = wn * 64 + (lane & 15);
  float *__restrict__ yl = args.y[pi] + (int64_t)(m0 + mb) * ldy + (n0 + nb);
  if (mrows == BM && nrows == BN) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float *__restrict__ yr = yl + (int64_t)(16 * a + r) * ldy;
#pragma unroll
        for (int b = 0; b < TN; ++b) __builtin_nontemporal_store(acc[a][b][r], yr + 16 * b);
      }
  } else {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (mb + 16 * a + r >= mrows) continue;
        float *__restrict__ yr = yl + (int64_t)(16 * a + r) * ldy;
#pragma unroll
        for (int b = 0; b < TN; ++b)
          if (nb + 16 * b < nrows) __builtin_nontemporal_store(acc[a][b][r], yr + 16 * b);
      }
  }
  if ((flags & kBadFlag) && drow_on && d_status) atomicOr(d_status, kDevInvalidByte);
}

void launch_chunk(const GemmBatch &args, int count, int64_t M, int64_t N, int64_t K, int G,
                  int64_t ldy, int32_t *d_status, hipStream_t stream) {
  const int64_t tpp = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)(tpp * count));
  if (G == 64)
    hipLaunchKernelGGL((gemm_kernel<64>), grid, dim3(NT), 0, stream, args, (int)M, (int)N, (int)K,
                       ldy, d_status);
  else
    hipLaunchKernelGGL((gemm_kernel<128>), grid, dim3(NT), 0, stream, args, (int)M, (int)N, (int)K,
                       ldy, d_status);
}

constexpr int64_t kChunkRows = int64_t(1) << 18;  // per launch: <= 2^22 blocks

}  // namespace

void launch_gemm(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t M,
                 int64_t N, int64_t K, int G, float *y, int32_t *d_status, hipStream_t stream) {
  if (gemm_wide_supported(1, M, N, K, G)) {
    launch_gemm_wide(1, &x, &packed, &scales, &y, M, N, K, d_status, stream);
    return;
  }
  const int64_t rowbytes = (K / G) * bytes_per_group(G);
  for (int64_t n_off = 0; n_off < N; n_off += kChunkRows) {
    const int64_t n_len = N - n_off < kChunkRows ? N - n_off : kChunkRows;
    for (int64_t m_off = 0; m_off < M; m_off += kChunkRows) {
      const int64_t m_len = M - m_off < kChunkRows ? M - m_off : kChunkRows;
      GemmBatch a;
      a.x[0] = x + m_off * K;
      a.packed[0] = packed + n_off * rowbytes;
      a.scales[0] = scales + n_off * (K / G);
      a.y[0] = y + m_off * N + n_off;
      launch_chunk(a, 1, m_len, n_len, K, G, N, d_status, stream);
    }
  }
}

void launch_gemm_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                         const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                         int64_t K, int G, int32_t *d_status, hipStream_t stream) {
  if (gemm_wide_supported(count, M, N, K, G)) {
    launch_gemm_wide(count, xs, packeds, scales, ys, M, N, K, d_status, stream);
    return;
  }
  // Same-shaped problems share a launch, kGemmMaxBatch at a time, while the
  // launch stays under 2^23 blocks; larger problems go one by one.
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (M > kChunkRows || N > kChunkRows || tiles * kGemmMaxBatch > (int64_t(1) << 23)) {
    for (int i = 0; i < count; ++i)
      launch_gemm(xs[i], packeds[i], scales[i], M, N, K, G, ys[i], d_status, stream);
    return;
  }
  for (int base = 0; base < count; base += kGemmMaxBatch) {
    const int n = count - base < kGemmMaxBatch ? count - base : kGemmMaxBatch;
    GemmBatch a;
    for (int i = 0; i < n; ++i) {
      a.x[i] = xs[base + i];
      a.packed[i] = packeds[base + i];
      a.scales[i] = scales[base + i];
      a.y[i] = ys[base + i];
    }
    launch_chunk(a, n, M, N, K, G, N, d_status, stream);
  }
}

// Problems of mixed shapes (shared M): one persistent launch for all of them
// when the 256 x 128 kernel takes every shape, else one batched launch per
// distinct (N, K), in order of first appearance.
void launch_gemm_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                         const uint16_t *const *scales, float *const *ys, int64_t M,
                         const int64_t *Ns, const int64_t *Ks, int G, int32_t *d_status,
                         hipStream_t stream) {
  if (gemm_wide_grouped_supported(count, M, Ns, Ks, G)) {
    launch_gemm_wide_grouped(count, xs, packeds, scales, ys, M, Ns, Ks, d_status, stream);
    return;
  }
  std::vector<char> done(count, 0);
  std::vector<const uint16_t *> gx, gs;
  std::vector<const uint8_t *> gp;
  std::vector<float *> gy;
  for (int i = 0; i < count; ++i) {
    if (done[i]) continue;
    gx.clear(); gs.clear(); gp.clear(); gy.clear();
    for (int j = i; j < count; ++j) {
      if (done[j] || Ns[j] != Ns[i] || Ks[j] != Ks[i]) continue;
      done[j] = 1;
      gx.push_back(xs[j]); gp.push_back(packeds[j]); gs.push_back(scales[j]); gy.push_back(ys[j]);
    }
    launch_gemm_batched((int)gx.size(), gx.data(), gp.data(), gs.data(), gy.data(), M, Ns[i],
                        Ks[i], G, d_status, stream);
  }
}

}  // namespace tq
