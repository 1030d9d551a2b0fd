// tq_gemm_wide.hip -- prefill matmul for gfx950 with 256-row activation
// tiles and 64-wide K stages (G = 128, M >= 256).
//
// y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
// (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation";
// prefill reuses each weight tile across many rows, "Revisit the Decode
// Roofline").
//
// Compared with gemm_kernel (128 x 128 tiles, 32-wide stages, two blocks per
// CU), a block here computes a 256 x 128 tile of y with 8 waves and owns the
// whole 160 KB of a CU's LDS:
//   * each decoded code is used by 256 activation rows instead of 128, so the
//     decode costs half as much per MFMA;
//   * a stage holds 32 MFMAs per wave between barriers instead of 16.
// Per 64-wide stage s:
//   - the activations of stage s+2 go from memory straight into their slot
//     of a 3-slot LDS ring (32 KB a slot; buffer loads with the lds modifier);
//   - the packed bytes of stage s+1, loaded two stages earlier into a
//     register ring, are looked up in the decode table, and the bytes of
//     stage s+3 are requested;
//   - the stage's 32 MFMAs per wave run (two 32-wide steps over 4 x 4 tiles
//     of v_mfma_f32_16x16x32_bf16 per wave), and the 16 codes each thread
//     decodes for stage s+1 are written to the other of two code slots;
//   - at the end of a group (every second stage) the group's fp32 partial is
//     scaled by s/2 and added to the accumulator;
//   - one barrier, after a wait that leaves the younger loads in flight.
// Codes enter the MFMA as the bf16 value 2c (exact, low byte zero: a pair of
// codes is one v_perm of table bytes), as in gemm_kernel.
// The kernel also takes the 2-bit format (four codes a byte, field c + 1,
// first code lowest: Avenue README, size note on 2-bit packing); only the
// table, the bytes a group and the way a run's codes are stitched differ.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>
#include <climits>

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
constexpr int G = 128;                  // this kernel's group size
// Weight formats: base-3 bytes (five codes a byte, 26 bytes a group) and
// 2-bit fields (four codes a byte, field c + 1, 32 bytes a group).
constexpr int kFmtBase3 = 0, kFmt2Bit = 1;
template <int FMT> struct Fmt;
template <> struct Fmt<kFmtBase3> { static constexpr int B = 26, CPB = 5; };
template <> struct Fmt<kFmt2Bit> { static constexpr int B = 32, CPB = 4; };
constexpr int BM = 256;                 // activation rows per block
constexpr int BN = 128;                 // weight rows per block
constexpr int NT = 512;                 // threads per block (8 waves)
constexpr int KS = 64;                  // K values per stage
constexpr int SPG = G / KS;             // stages per group: 2
constexpr int XRING = 3;                // activation slots
constexpr int XSLOT = BM * KS * 2;      // 32 KiB
constexpr int CSLOT = BN * KS * 2;      // 16 KiB
constexpr int kCopies = 16;
constexpr int kEntryBytes = 8;
constexpr int LUTB = 256 * kCopies * kEntryBytes;  // 32 KiB
constexpr uint32_t kCsOff = XRING * XSLOT;
constexpr uint32_t kLutOff = kCsOff + 2 * CSLOT;
constexpr int SMEM = kLutOff + LUTB;    // 160 KiB: the whole LDS of a CU
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr uint32_t kBadFlag = 0xFF00u;  // in the high dword of invalid bytes' entries
constexpr int TM = 4, TN = 4;           // 16 x 16 tiles per wave: 64 x 64

// Problems of one launch (M is shared): their pointers, ordered by shape,
// and up to kWideMaxShapes shapes (N, K).  The problems of shape g are
// first[g], first[g] + 1, ...; their tiles start at tile t0[g] of the launch
// (t0 of an absent shape: INT_MAX) and follow one another problem by
// problem.  The tile -> problem lookup is a fixed number of comparisons: a
// loop there would put branches in every stage.  Tile walk: block b takes
// tiles b, b + grid, ... (skip = 0).  With skip > 0 the `heavy` first blocks,
// which draw one more tile of the longest shape (lead + 1 against lead), let
// the others take the first `skip` rounds of the remaining tiles alone, so
// that the blocks' shares of stages come out closer to equal.
constexpr int kWideMaxBatch = 128;
constexpr int kWideMaxShapes = 4;
struct WideBatch {
  const uint16_t *x[kWideMaxBatch];
  const uint8_t *packed[kWideMaxBatch];
  const uint16_t *scales[kWideMaxBatch];
  float *y[kWideMaxBatch];
  int n[kWideMaxShapes], k[kWideMaxShapes], tpp[kWideMaxShapes], first[kWideMaxShapes];
  int t0[kWideMaxShapes];
  int total;
  int heavy, lead, skip;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Byte offset of 16-byte chunk kc (0..7) of row r in a swizzled tile of
// 128-byte rows.  16 consecutive rows reading one chunk, and 16 consecutive
// rows writing one chunk, land in 16 different 16-byte bank groups.
__device__ __forceinline__ uint32_t swz(uint32_t r, uint32_t kc) {
  return 16u * (8u * r + (kc ^ ((r >> 1) & 7u)));
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

// Table entry for a byte of 2-bit fields (field i = c_i + 1, first code
// lowest): high bytes of 2*c_i, i = 0..3, in the low dword; the flag in the
// high dword when a field is 3 (invalid; its code counts as 0).
__device__ __forceinline__ u32x2 code_entry2(uint32_t e) {
  uint32_t lo = 0u, bad = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t f = (e >> (2 * i)) & 3u;
    lo |= (f == 0u ? 0xC0u : (f == 2u ? 0x40u : 0u)) << (8 * i);
    bad |= f == 3u ? kBadFlag : 0u;
  }
  return u32x2{lo, bad};
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

// The same for a run of 16 2-bit codes: four whole bytes, four codes each.
__device__ __forceinline__ void stitch2(const uint32_t (&lo)[4], uint32_t (&out)[8]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t b1 = 2u * (uint32_t)(w & 1), b2 = b1 + 1u;
    out[w] = __builtin_amdgcn_perm(lo[w >> 1], lo[w >> 1], 0x000C000Cu | (b1 << 8) | (b2 << 24));
  }
}

template <int V>
struct Int {
  static constexpr int value = V;
};

// A tile of one problem: rows [m0, m0 + mrows) of x, rows [n0, n0 + nrows)
// of W, and the problem's N and K.  Tile j of a block is tile blockIdx.x +
// j * gridDim.x of the launch (problem-major); past the launch's tiles it is
// empty (no rows: every load of it reads zeros; K = one group).
struct Tile {
  int pi, m0, n0, mrows, nrows, N, K;
};

// Tile index of the j-th tile of this block (see WideBatch).
__device__ __forceinline__ int walk_tile(const WideBatch &a, int j) {
  const int b = (int)blockIdx.x, grid = (int)gridDim.x;
  if (a.skip == 0) return b + j * grid;
  const bool heavy = b < a.heavy;
  const int jl = a.lead + (heavy ? 1 : 0);  // this block's tiles of the longest shape
  if (j < jl) return b + j * grid;
  const int light = grid - a.heavy;
  const int v = j - jl + (heavy ? a.skip : 0);  // round among the remaining tiles
  return v < a.skip ? a.t0[1] + v * light + (b - a.heavy)
                    : a.t0[1] + a.skip * light + (v - a.skip) * grid + b;
}

// Tiles of this block.
__device__ __forceinline__ int walk_count(const WideBatch &a) {
  const int b = (int)blockIdx.x, grid = (int)gridDim.x;
  if (a.skip == 0) return (a.total - b + grid - 1) / grid;
  const bool heavy = b < a.heavy;
  const int rest0 = a.t0[1] + a.skip * (grid - a.heavy);  // first tile of the shared rounds
  const int left = a.total - rest0 - b;
  return a.lead + (heavy ? 1 : a.skip) + (left > 0 ? (left + grid - 1) / grid : 0);
}

__device__ __forceinline__ Tile block_tile(const WideBatch &a, int j, int M, int tilesM) {
  const int t = walk_tile(a, j);
  Tile r;
  if (t >= a.total) {
    r.pi = 0; r.m0 = 0; r.n0 = 0; r.mrows = 0; r.nrows = 0; r.N = 0; r.K = G;
    return r;
  }
  static_assert(kWideMaxShapes == 4, "the shape lookup below compares against t0[1..3]");
  const int g = (int)(t >= a.t0[1]) + (int)(t >= a.t0[2]) + (int)(t >= a.t0[3]);
  const int tg = t - a.t0[g], tpp = a.tpp[g];
  const int q = tg / tpp;
  r.pi = a.first[g] + q;
  r.N = a.n[g];
  r.K = a.k[g];
  const int tt = tg - q * tpp;
  r.m0 = (tt % tilesM) * BM;
  r.n0 = (tt / tilesM) * BN;
  r.mrows = min(BM, M - r.m0);
  r.nrows = min(BN, r.N - r.n0);
  return r;
}

// Persistent blocks, one per CU: block b computes tiles b, b + grid, ... one
// after another.  The stage pipeline (activations two stages ahead, packed
// bytes three, scales one group) runs on across tile boundaries: each of the
// three load streams keeps its own tile and moves to the next tile when its
// stage count wraps, so a tile's first stages are loaded while the previous
// tile computes, and the table is built once per block.  FMT: the weight
// format (kFmtBase3 or kFmt2Bit).
template <int FMT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
// `args` is the first kernel argument only to lay the table out at the start of
// the argument segment, where the body reads it.
void gemm_wide_kernel(const WideBatch args, int M, int32_t *__restrict__ d_status) {
  constexpr int B = Fmt<FMT>::B, CPB = Fmt<FMT>::CPB;
  (void)args;
  __shared__ __align__(16) unsigned char smem_raw[SMEM];
  lds_bytes *smem = (lds_bytes *)smem_raw;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int wm = wv >> 1, wn = wv & 1;
  const int tilesM = (M + BM - 1) / BM;
  // The problem table is read through the kernel-argument segment pointer:
  // indexing the by-value struct with a computed shape index makes the
  // compiler copy it to scratch memory.
  const WideBatch &args_ = *reinterpret_cast<const WideBatch *>(
      (const void *)__builtin_amdgcn_kernarg_segment_ptr());
  const int ntiles = walk_count(args_);
  auto tile = [&](int j) { return block_tile(args_, j, M, tilesM); };

  // ---- decode table: two threads per entry, eight copies each, the copy
  // index rotated by the entry to spread the banks ----
  {
    const uint32_t e = (uint32_t)tid & 255u, half = (uint32_t)tid >> 8;
    const u32x2 v = FMT == kFmtBase3 ? code_entry(e) : code_entry2(e);
#pragma unroll
    for (int k = 0; k < kCopies / 2; ++k) {
      const uint32_t j = (8u * half + (uint32_t)k + e) & (kCopies - 1);
      *(lds_u32x2 *)(smem + kLutOff + (e * kCopies + j) * kEntryBytes) = v;
    }
  }

  // Every stage issues the same loads -- past the end they read junk or
  // zeros into slots that are never consumed -- so the wait counts are fixed.
  const uint32_t wvs = __builtin_amdgcn_readfirstlane(wv);  // wave index, scalar

  // ---- activation stream: op i of thread t fills chunk 512 i + t of a slot
  // (row r = chunk / 8).  Offsets stay in the per-lane offset, the only part
  // of a raw buffer address that is range-checked. ----
  // The row of op i is r0 + 64 i, with the same swizzled chunk for every i.
  const uint32_t xr0 = (uint32_t)tid >> 3;
  const uint32_t xchunk = (((uint32_t)tid & 7u) ^ ((xr0 >> 1) & 7u)) * 8u;
  int jx = 0, sx = 0, ux = 0;  // tile, its stage, ring slot of the next request
  int xrows = 0;               // rows of the stream's tile
  uint32_t xK = 0, xbase = 0;  // its K, and this thread's offset in its first stage
  int xnS = 1;                 // its stages
  __amdgpu_buffer_rsrc_t rx;
  auto set_x = [&](int j) {
    const Tile T = tile(j);
    rx = make_rsrc(args_.x[T.pi] + (int64_t)T.m0 * T.K, (uint32_t)T.mrows * (uint32_t)T.K * 2u);
    xrows = T.mrows;
    xK = (uint32_t)T.K;
    xnS = T.K / KS;
    xbase = (xr0 * xK + xchunk) * 2u;
  };
  set_x(0);
  auto dma_x = [&]() {
    const uint32_t slot = (uint32_t)ux * XSLOT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lds_bytes *dst = smem + slot + 16u * (512u * i + 64u * wvs);
      const uint32_t off = (int)(xr0 + 64u * i) < xrows
                               ? xbase + (uint32_t)i * (64u * 2u) * xK + (uint32_t)sx * (KS * 2)
                               : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void *)dst,
                                               16, off, 0, 0, 0);
    }
    ux = ux == XRING - 1 ? 0 : ux + 1;
    if (++sx == xnS) {
      sx = 0;
      set_x(++jx);
    }
  };

  // ---- scale stream: lanes hold column n = wn*64 + tn*16 + (lane & 15) ----
  const int sn0 = wn * 64 + (lane & 15);  // column of op tn: sn0 + 16 tn
  int js = 0, gs = 0;  // tile, its group
  int srows = 0;       // rows of the stream's tile
  int snG = 1;         // its groups per row
  __amdgpu_buffer_rsrc_t rs;
  auto set_s = [&](int j) {
    const Tile T = tile(j);
    snG = T.K / G;
    rs = make_rsrc(args_.scales[T.pi] + (int64_t)T.n0 * snG, (uint32_t)T.nrows * (uint32_t)snG * 2u);
    srows = T.nrows;
  };
  set_s(0);
  uint32_t sc_cur[TN], sc_next[TN];
  auto load_scales = [&](uint32_t (&dst)[TN]) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int n = sn0 + 16 * tn;
      const uint32_t off = n < srows ? 2u * ((uint32_t)n * (uint32_t)snG + (uint32_t)gs) : kOutOfRange;
      dst[tn] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
    }
    if (++gs == snG) {
      gs = 0;
      set_s(++js);
    }
  };

  // ---- packed-byte stream: thread (row dr, quarter dq) decodes codes 16 dq
  // .. 16 dq + 15 of each stage; two dwords hold the run's four bytes ----
  const int dr = tid & (BN - 1);
  const uint32_t dqs = __builtin_amdgcn_readfirstlane(tid >> 7);  // uniform over a wave
  int jp = 0, sp = 0;  // tile, its stage
  __amdgpu_buffer_rsrc_t rp;
  uint32_t prow;
  int pnS = 1;  // stages of the stream's tile
  auto set_p = [&](int j) {
    const Tile T = tile(j);
    const uint32_t rowbytes = (uint32_t)(T.K / G) * B;
    pnS = T.K / KS;
    const uintptr_t pabs =
        reinterpret_cast<uintptr_t>(args_.packed[T.pi]) + (uint64_t)T.n0 * rowbytes;
    const uint32_t pbase = (uint32_t)(pabs & 3u);  // packed has any alignment
    // The range is a whole number of dwords, so a dword load is either fully
    // in range or fully past it (then it reads 0).
    rp = make_rsrc(reinterpret_cast<const void *>(pabs - pbase),
                   (pbase + (uint32_t)T.nrows * rowbytes + 3u) & ~3u);
    prow = dr < T.nrows ? pbase + (uint32_t)dr * rowbytes : kOutOfRange;
  };
  set_p(0);
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

  // ---- MFMA operands: lane reads rows r0 + 16 a, chunk 4 ks + (lane >> 4) ----
  const uint32_t kq = (uint32_t)(lane >> 4);
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    aoff[ks] = swz((uint32_t)(wm * 64 + (lane & 15)), 4u * ks + kq);
    boff[ks] = kCsOff + swz((uint32_t)(wn * 64 + (lane & 15)), 4u * ks + kq);
  }

  f32x4 acc[TM][TN], part[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      part[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // ---- epilogue of tile j: lane holds column (lane & 15), rows
  // 4*(lane>>4) + r of each 16 x 16 tile; y is written with nontemporal
  // stores (never read back here; 3% faster on the FFN stack at M = 2048) ----
  auto store_tile = [&](int j) {
    const Tile T = tile(j);
    const int mb = wm * 64 + 4 * (lane >> 4), nb = wn * 64 + (lane & 15);
    const int64_t ldy = T.N;
    float *__restrict__ yl = args_.y[T.pi] + (int64_t)(T.m0 + mb) * ldy + (T.n0 + nb);
    if (T.mrows == BM && T.nrows == BN) {
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
          if (mb + 16 * a + r >= T.mrows) continue;
          float *__restrict__ yr = yl + (int64_t)(16 * a + r) * ldy;
#pragma unroll
          for (int b = 0; b < TN; ++b)
            if (nb + 16 * b < T.nrows) __builtin_nontemporal_store(acc[a][b][r], yr + 16 * b);
        }
    }
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // The rest is instantiated per decode quarter DQ (uniform over a wave), so
  // that each stage is one block the scheduler can interleave.
  auto body = [&](auto dqc) {
    constexpr int DQ = decltype(dqc)::value;
    // one 8-byte load (one count of vmcnt) from the dword holding the run's
    // first byte
    auto load_packed = [&](uint32_t (&dst)[2], uint32_t &ofs) {
      const uint32_t a = prow + (uint32_t)((sp >> 1) * B) +
                         ((sp & 1) ? (uint32_t)((KS + 16 * DQ) / CPB) : (uint32_t)(16 * DQ / CPB));
      ofs = a & 3u;
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rp, a & ~3u, 0, 0);
      dst[0] = v.x;
      dst[1] = v.y;
      if (++sp == pnS) {
        sp = 0;
        set_p(++jp);
      }
    };
    // codes of a run that is stage ST of its group -> two chunks of slot cs
    auto emit = [&](auto stc, const uint32_t (&lo)[4], const uint32_t (&hi)[4], uint32_t cs) {
      constexpr int ST = decltype(stc)::value;
      flags |= (hi[0] | hi[1]) | (hi[2] | hi[3]);
      uint32_t out[8];
      if constexpr (FMT == kFmtBase3)
        stitch<(ST * KS + 16 * DQ) % 5>(lo, hi, out);
      else
        stitch2(lo, out);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *(lds_u32x4 *)(smem + cs + swz((uint32_t)dr, (uint32_t)(2 * DQ + i))) =
            u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
    };

    // ---- prologue: all of it completes before the loop, so the compiler's
    // wait counts inside the loop need not cover it ----
    uint32_t ring[2][2], rofs[2], first[2], first_ofs;
    load_scales(sc_cur);
    dma_x();
    dma_x();
    load_packed(first, first_ofs);
    load_packed(ring[1], rofs[1]);
    load_packed(ring[0], rofs[0]);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    __syncthreads();                // table and stage 0 activations ready
    {
      uint32_t lo[4], hi[4];
      lookup(first, first_ofs, lo, hi);
      emit(Int<0>{}, lo, hi, kCsOff);
    }
    __syncthreads();

    int uc = 0;  // ring slot of the stage being computed
    int sc = 0;  // its stage within its tile
    int jc = 0;  // its tile
    int cnS = tile(0).K / KS;  // its tile's stages
    // a stage is stage ST (= its index & 1) of its group; it reads code slot
    // ST and the activation slot uc
    auto stage = [&](auto stc) {
      constexpr int ST = decltype(stc)::value;
      constexpr int P = ST, Q = 1 - ST;
      constexpr int ST1 = (ST + 1) % SPG;  // place of the next stage in its group
      const uint32_t xs = (uint32_t)uc * XSLOT;
      // operands of one 32-wide step: 4 activation and 4 code fragments
      auto read_ops = [&](int ks, bf16x8 (&av)[TM], bf16x8 (&bv)[TN]) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
          av[a] = *(lds_bf16x8_c *)(smem + xs + aoff[ks] + 2048u * a);
#pragma unroll
        for (int b = 0; b < TN; ++b)
          bv[b] = *(lds_bf16x8_c *)(smem + P * CSLOT + boff[ks] + 2048u * b);
      };
      auto mfmas = [&](int ks, const bf16x8 (&av)[TM], const bf16x8 (&bv)[TN]) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            part[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                av[a], bv[b], (ST == 0 && ks == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : part[a][b], 0,
                0, 0);
      };
      bf16x8 av0[TM], bv0[TN], av1[TM], bv1[TN];
      read_ops(0, av0, bv0);
      // table lookups for the next stage, after this stage's first operand
      // reads so that the first MFMAs wait for those only: its bytes were
      // requested two stages ago (past the last stage they decode junk into
      // the free code slot)
      uint32_t lo[4], hi[4];
      lookup(ring[Q], rofs[Q], lo, hi);
      if (ST == 0) load_scales(sc_next);
      dma_x();
      load_packed(ring[Q], rofs[Q]);
      // the next stage's codes, assembled and written between the first MFMAs
      emit(Int<ST1>{}, lo, hi, kCsOff + (uint32_t)Q * CSLOT);
      mfmas(0, av0, bv0);
      read_ops(1, av1, bv1);
      mfmas(1, av1, bv1);
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
      // Instruction order for the scheduler: the operand and table reads and
      // the loads first, then each MFMA followed by vector-ALU work -- the
      // code assembly after the first seven, the scaling after the rest -- so
      // that the decode and the scaling run in the MFMA shadow.
      constexpr int kValu = ST == SPG - 1 ? 3 : 1;
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // VALU: addresses
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // DS reads: step 0, then table
      __builtin_amdgcn_sched_group_barrier(0x020, 10, 0);  // VMEM reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        if (i < 7)
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU: code assembly
        else
          __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
        if (i == 3) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // DS reads: step 1
        if (i == 7) __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);  // DS writes
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
      }
      uc = uc == XRING - 1 ? 0 : uc + 1;
      if (ST == SPG - 1 && sc == cnS - 1) {
        // last stage of a tile: store it, then a full wait (the stores count
        // in vmcnt too) before the barrier
        store_tile(jc);
        ++jc;
        sc = 0;
        cnS = tile(jc).K / KS;
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        return;
      }
      ++sc;
      // The activations of the next stage (requested during the previous
      // stage) must have landed before the barrier.  Only this stage's loads
      // may stay in flight -- its scales (4, first stage of a group only),
      // activations (4) and bytes (1) -- whatever order the compiler gave the
      // previous stage's loads.
      if (ST == 0)
        asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    int nstages = 0;  // a multiple of SPG
    for (int j = 0; j < ntiles; ++j) nstages += tile(j).K / KS;
    for (int u = 0; u < nstages; u += SPG) {
      stage(Int<0>{});
      stage(Int<1>{});
    }
  };
  switch (dqs) {
    case 0: body(Int<0>{}); break;
    case 1: body(Int<1>{}); break;
    case 2: body(Int<2>{}); break;
    default: body(Int<3>{}); break;
  }
  // no load may still be writing this block's LDS when it exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if ((flags & kBadFlag) && d_status) atomicOr(d_status, kDevInvalidByte);
}

}  // namespace

bool gemm_wide_supported(int count, int64_t M, int64_t N, int64_t K, int G_) {
  // G = 128 and at least one whole 256-row tile; 32-bit offsets (a 256-row
  // slab of x); and enough tiles to give at least 3/4 of the 256 CUs one
  // block each -- smaller grids run faster as 128 x 128 tiles, two per CU
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return G_ == G && M >= BM && K % G == 0 && tiles * kWideMaxBatch < (int64_t(1) << 30) &&
         (int64_t)BM * K * 2 < (int64_t(1) << 31) && tiles * count >= 192;
}

bool gemm_wide_grouped_supported(int count, int64_t M, const int64_t *Ns, const int64_t *Ks,
                                 int G_) {
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) {
    if (!gemm_wide_supported(1 << 20, M, Ns[i], Ks[i], G_)) return false;
    tiles += ((M + BM - 1) / BM) * ((Ns[i] + BN - 1) / BN);
  }
  return tiles >= 192 && tiles < (int64_t(1) << 30);
}

// The tile walk of a launch (WideBatch): when the tiles of the longest shape
// do not split evenly over the blocks, the number of rounds of the remaining
// tiles that the blocks with one more long tile skip, chosen to minimise the
// largest block's stages (each tile counted by its K), 0 if none helps.
// Tiles are ordered by K, longest first, so within each class of blocks
// (one more long tile, or not) the first block draws the most and the
// costliest tiles: the walk is simulated for blocks 0 and `heavy` only.
static void plan_walk(WideBatch &a, int grid) {
  a.heavy = 0; a.lead = 0; a.skip = 0;
  if (a.t0[1] == INT_MAX || grid <= 0) return;  // one shape
  const int L = a.t0[1], heavy = L % grid;
  if (heavy == 0) return;
  const int light = grid - heavy, cap = (a.total - L) / light;
  auto cost_of = [&](int t) {
    const int g = (int)(t >= a.t0[1]) + (int)(t >= a.t0[2]) + (int)(t >= a.t0[3]);
    return (int64_t)a.k[g];
  };
  auto load_of = [&](int b, int d) {
    const bool hv = b < heavy;
    const int jl = L / grid + (hv ? 1 : 0);
    int64_t sum = 0;
    for (int j = 0;; ++j) {
      int t;
      if (d == 0 || j < jl) {
        t = b + j * grid;
      } else {
        const int v = j - jl + (hv ? d : 0);
        t = v < d ? L + v * light + (b - heavy) : L + d * light + (v - d) * grid + b;
      }
      if (t >= a.total) break;
      sum += cost_of(t);
    }
    return sum;
  };
  int64_t best = -1;
  int best_d = 0;
  for (int d = 0; d <= cap && d <= 16; ++d) {
    const int64_t l0 = load_of(0, d), l1 = load_of(heavy, d);
    const int64_t mx = l0 > l1 ? l0 : l1;
    if (best < 0 || mx < best) { best = mx; best_d = d; }
  }
  if (best_d > 0) { a.heavy = heavy; a.lead = L / grid; a.skip = best_d; }
}

// Launches of up to kWideMaxBatch problems and kWideMaxShapes shapes, one
// persistent block per CU.  Shapes are placed longest K first, so that the
// blocks' round-robin share of the tiles ends with the short ones.
static void launch_wide_fmt(int fmt, int count, const uint16_t *const *xs,
                            const uint8_t *const *packeds, const uint16_t *const *scales,
                            float *const *ys, int64_t M, const int64_t *Ns, const int64_t *Ks,
                            int32_t *d_status, hipStream_t stream) {
  auto kernel = fmt == kFmtBase3 ? gemm_wide_kernel<kFmtBase3> : gemm_wide_kernel<kFmt2Bit>;
  static int cus[64] = {};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  // problems by shape: K descending, then N descending, then in order
  std::vector<int> order(count);
  for (int i = 0; i < count; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return Ks[a] != Ks[b] ? Ks[a] > Ks[b] : Ns[a] > Ns[b];
  });
  const int64_t tilesM = (M + BM - 1) / BM;
  WideBatch a;
  int n = 0, shapes = 0;
  auto flush = [&]() {
    if (n == 0) return;
    for (int g = shapes; g < kWideMaxShapes; ++g) {
      a.n[g] = 0; a.k[g] = G; a.tpp[g] = 1; a.first[g] = n; a.t0[g] = INT_MAX;
    }
    const int grid = a.total < cus[dev] ? a.total : cus[dev];
    plan_walk(a, grid);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NT), 0, stream, a, (int)M, d_status);
    n = 0;
    shapes = 0;
  };
  for (int i = 0; i < count; ++i) {
    const int p = order[i];
    const bool new_shape = shapes == 0 || Ns[p] != a.n[shapes - 1] || Ks[p] != a.k[shapes - 1];
    if (n == kWideMaxBatch || (new_shape && shapes == kWideMaxShapes)) flush();
    if (shapes == 0 || Ns[p] != a.n[shapes - 1] || Ks[p] != a.k[shapes - 1]) {
      const int g = shapes++;
      a.n[g] = (int)Ns[p];
      a.k[g] = (int)Ks[p];
      a.tpp[g] = (int)(tilesM * ((Ns[p] + BN - 1) / BN));
      a.first[g] = n;
      a.t0[g] = g == 0 ? 0 : a.total;
      if (g == 0) a.total = 0;
    }
    a.x[n] = xs[p];
    a.packed[n] = packeds[p];
    a.scales[n] = scales[p];
    a.y[n] = ys[p];
    ++n;
    a.total += a.tpp[shapes - 1];
  }
  flush();
}

void launch_gemm_wide_grouped(int count, const uint16_t *const *xs,
                              const uint8_t *const *packeds, const uint16_t *const *scales,
                              float *const *ys, int64_t M, const int64_t *Ns, const int64_t *Ks,
                              int32_t *d_status, hipStream_t stream) {
  launch_wide_fmt(kFmtBase3, count, xs, packeds, scales, ys, M, Ns, Ks, d_status, stream);
}

void launch_gemm_wide(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                      const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                      int64_t K, int32_t *d_status, hipStream_t stream) {
  std::vector<int64_t> Ns(count, N), Ks(count, K);
  launch_wide_fmt(kFmtBase3, count, xs, packeds, scales, ys, M, Ns.data(), Ks.data(), d_status,
                  stream);
}

void launch_gemm2_wide(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                       const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                       int64_t K, int32_t *d_status, hipStream_t stream) {
  std::vector<int64_t> Ns(count, N), Ks(count, K);
  launch_wide_fmt(kFmt2Bit, count, xs, packeds, scales, ys, M, Ns.data(), Ks.data(), d_status,
                  stream);
}

}  // namespace tq
