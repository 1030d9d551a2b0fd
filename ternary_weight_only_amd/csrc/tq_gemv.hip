// tq_gemv.hip -- skinny matmul (2 <= M <= 16, and M = 1 for shapes the M = 1
// kernel in tq_gemv_m1.hip does not take) for gfx950.
//
// y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
// (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation":
// the group scale multiplies the group's inner sum; fp32 accumulation.
// "Revisit the Decode Roofline": a decode with few activation rows streams
// every packed weight once, so the kernel is bound by HBM bandwidth).
//
// The multiply-adds run on the matrix cores (v_mfma_f32_16x16x32_bf16), one
// packed byte per lane and MFMA:
//   * The 32 k-slots of an MFMA are four bytes' worth of codes, 8 slots per
//     byte: the byte's five codes and three zeros.  Lane l = j + 16 q feeds
//     byte (T q + t) of the current group of weight row j of a 16-row tile
//     (B operand) and the five matching activations of x row j (A operand;
//     rows j >= M are zero), so after T MFMAs (T = 8 for G=128, 4 for G=64)
//     lane (j, q) holds the group's partial sums y[4q + r][row j], r = 0..3.
//   * A 256-entry LDS table maps a byte to exactly that B fragment: three
//     bf16 code pairs (c0,c1)(c2,c3)(c4,0) and a zero dword.  One
//     ds_read_b128 per byte, no decode arithmetic.  The table is replicated
//     16 times, copy j in bank group j, and lane l reads copy l % 16; the
//     address (byte * 256 + copy * 16) is one v_perm_b32.  Entries 243..255
//     are NaN, so an invalid byte makes its outputs NaN.  Inf activations or
//     fp32 overflow can give NaN too, so a NaN output only marks its weight
//     row: the row's bytes are scanned when it is stored, and only a byte
//     >= 243 sets the invalid-byte status.
//   * Byte slots past the group's ceil(G/5) bytes (and code positions past G)
//     meet zero activations, so the padding trits and the neighbouring
//     group's bytes contribute nothing.
//   * A group's partial tile is scaled by its fp16 scale in fp32 and added
//     to the accumulator.
// Work: a wave's tile is R consecutive 16-row MFMA tiles (R = 1, 2 or 4):
// the activation fragments of a group are built once and feed the MFMAs of
// all R, so the activations are read once per 16R weight rows.  A block of
// 8 waves takes "chunks" of TB consecutive tiles (over the problems of the
// launch), with the K groups of each tile split into S contiguous parts
// (TB * S = 8): wave (a, p) computes part p of tile a of each chunk.  Every wave runs the same number of group iterations per
// chunk (ceil(nG / S); past its part a wave reads zeros), so the block
// reaches each chunk's end together; the S partial tiles are then added
// through LDS in a fixed order (deterministic results) and stored.  Within a
// chunk a wave issues the packed bytes and scales of up to BR groups at
// once, and the activations two groups ahead (see the main loop for why the
// two streams are issued in that order).  The blocks are persistent (one per
// CU: the kernel takes up to 256 registers a lane at two waves a SIMD, so all
// are resident at once) and take chunks b, b + grid, ...
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 8;          // waves per block
constexpr int kThreads = kWave * kWaves;
constexpr int kCopies = 16;        // table replicas, one per 16-byte LDS bank group
constexpr int kLutEntries = 256;   // byte values; 243..255 decode to NaN
constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past any range: loads give 0
constexpr int kMaxBatch = 64;      // problems per batched launch
constexpr int kXLead = 2;          // group iterations of activations in flight per wave
constexpr int kXBuf = 4;           // activation buffers (> kXLead)
constexpr int kMaxBlocks = 256;    // one 8-wave block per CU (two waves a SIMD)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4_c;
typedef __attribute__((address_space(3))) const unsigned char lds_bytes_c;

// Table entry for byte value e: three bf16 pairs of the codes of its five
// base-3 digits (first weight = least significant digit), fourth dword 0.
__device__ __forceinline__ uint4 lut_entry(uint32_t e) {
  if (e >= 243u) return make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0u);
  uint32_t h[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t d = e % 3u;
    e /= 3u;
    h[i] = d == 0u ? 0xBF80u : (d == 2u ? 0x3F80u : 0u);  // code -1, 0, +1 in bf16
  }
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4], 0u);
}

// 1 if one of the `len` bytes at p is >= 243 (an invalid base-3 byte); the
// rare path of a NaN output.
__device__ __attribute__((noinline)) uint32_t row_has_invalid_byte(const uint8_t *p,
                                                                  uint32_t len) {
  for (uint32_t i = 0; i < len; ++i)
    if (p[i] >= 243u) return 1u;
  return 0u;
}

// Buffer resource over [p, p + bytes): the hardware range check returns 0 for
// a load past `bytes`, so loads need no branches at the edges.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Up to kMaxBatch same-shaped problems per launch, passed by value.
struct GemvBatch {
  const uint16_t *x[kMaxBatch];
  const uint8_t *packed[kMaxBatch];
  const uint16_t *scales[kMaxBatch];
  float *y[kMaxBatch];
};

template <int G>
struct Geo {
  static constexpr int B = bytes_per_group(G);  // 13 or 26 bytes per group
  static constexpr int T = G == 128 ? 8 : 4;    // bytes per k-lane per group (= MFMAs per tile)
  static constexpr int PD = T == 8 ? 3 : 2;     // packed dwords a lane loads per group
  static constexpr int XL = 5;                  // activation loads per lane per group
  static constexpr int XW = G == 128 ? 4 : 2;   // dwords per activation load
};

template <int G, int BR, int R>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemv_kernel(const GemvBatch args, int count, int M, int N, int K, int lgS, int nchunks,
                 int64_t ldy, int32_t *__restrict__ d_status) {
  using Gm = Geo<G>;
  constexpr int T = Gm::T, PD = Gm::PD, B = Gm::B, XL = Gm::XL, XW = Gm::XW;
  __shared__ uint4 lut[kLutEntries * kCopies];
  __shared__ f32x4 red[kWaves][kWave];

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = 1 << lgS, TB = kWaves >> lgS;
  const int part = wv & (S - 1), slot = wv >> lgS;   // K part and tile slot of the wave
  const int nG = K / G;
  const int ngw = (nG + S - 1) >> lgS;                // group iterations per chunk
  const int g_begin = part * ngw;                     // the wave's first group (may be >= nG)
  const uint32_t rowbytes = (uint32_t)nG * B;
  constexpr int TR = 16 * R;                          // rows of a wave's tile: R MFMA tiles
  const int tpp = (N + TR - 1) / TR;                  // tiles per problem
  const int ntiles = tpp * count;
  const int bid = (int)blockIdx.x, grid = (int)gridDim.x;
  const int mychunks = nchunks > bid ? (nchunks - bid + grid - 1) / grid : 0;


  const int j = lane & 15, q = lane >> 4;
  const uint32_t copyoff = (uint32_t)j * 16u;  // byte 0 of a perm source: the lane's table copy
  // Lanes q = 3 run past the group's last byte (slots 26..31 of 32 for
  // G=128, 13..15 of 16 for G=64): those slots are forced to byte 121, whose
  // codes are all 0, so whatever follows the group cannot turn into NaN.
  constexpr int kLive3 = B - 3 * T;  // live bytes of lane q = 3: 2 or 1
  const uint32_t keep = q == 3 ? (kLive3 == 2 ? 0x0000FFFFu : 0x000000FFu) : 0xFFFFFFFFu;
  const uint32_t wmask[2] = {keep, q == 3 ? 0u : 0xFFFFFFFFu};
  const uint32_t wfill[2] = {0x79797979u & ~keep, q == 3 ? 0x79797979u : 0u};
  lds_bytes_c *lut_bytes = (lds_bytes_c *)(lut);

  // Activations of lane (j, q) for a group: x[j][gG + 5Tq .. gG + 5Tq + 5T),
  // as XL loads of XW dwords at offsets aligned to their size (none
  // straddles the end of x); for q = 3 only the first load holds positions
  // < G, the others read zeros (code positions past G carry no activation).
  uint32_t xoff[XL];
#pragma unroll
  for (int u = 0; u < XL; ++u) {
    const bool on = j < M && !(q == 3 && u >= 1);
    xoff[u] = on ? ((uint32_t)j * (uint32_t)K + (uint32_t)(5 * T * q) + (uint32_t)(XW * 2 * u)) * 2u
                 : kOutOfRange;
  }

  // Tile of the wave in chunk k of the block: TR = 16 R weight rows, R MFMA
  // tiles that share the activations; past the block's chunks or the
  // launch's tiles it has no rows (every load of it reads zeros).
  struct Tile {
    int pi, row0, nrows;
  };
  auto tile_of = [&](int k) -> Tile {
    const int t = (bid + k * grid) * TB + slot;
    if (k >= mychunks || t >= ntiles) return Tile{0, 0, 0};
    const int pi = t / tpp;
    const int row0 = (t - pi * tpp) * TR;
    return Tile{pi, row0, min(TR, N - row0)};
  };

  struct PkStage {
    uint32_t pk[R][PD];
    uint32_t sc[R];
    uint32_t ofs[R];
  };
  struct XStage {
    uint32_t xd[XL * XW];
  };
  // A load stream's position: chunk k of the block, group iteration gi, and
  // the tile's buffer descriptors, rebuilt only when the stream moves to the
  // next chunk (the problem's pointers are read from the kernel arguments
  // there, not per load).
  struct PkCursor {
    int k, nrows;
    uint32_t pbase;
    __amdgpu_buffer_rsrc_t rp, rs;
  };
  struct XCursor {
    int k, nrows;
    __amdgpu_buffer_rsrc_t rx;
  };
  auto set_pk = [&](PkCursor &c) {
    const Tile w = tile_of(c.k);
    const uintptr_t pabs =
        reinterpret_cast<uintptr_t>(args.packed[w.pi]) + (uint64_t)w.row0 * rowbytes;
    c.pbase = (uint32_t)(pabs & 3u);
    c.nrows = w.nrows;
    // whole dwords: a dword load is fully in range or fully past it (reads 0)
    c.rp = make_rsrc(reinterpret_cast<const void *>(pabs - c.pbase),
                     (c.pbase + (uint32_t)w.nrows * rowbytes + 3u) & ~3u);
    c.rs = make_rsrc(args.scales[w.pi] + (int64_t)w.row0 * nG,
                     (uint32_t)w.nrows * (uint32_t)nG * 2u);
  };
  auto set_x = [&](XCursor &c) {
    const Tile w = tile_of(c.k);
    c.nrows = w.nrows;
    c.rx = make_rsrc(args.x[w.pi], (uint32_t)M * (uint32_t)K * 2u);
  };
  // packed bytes and scale of group iteration gi of the cursor's tile (rows
  // past its rows, groups past nG and iterations past the burst (!live)
  // read 0: scale 0 and zero activations add nothing)
  auto issue_pk = [&](const PkCursor &c, int gi, bool live, PkStage &st) {
    const int g = g_begin + gi;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = 16 * r + j;  // the lane's row within the tile
      const bool on = live && row < c.nrows && g < nG;
      const uint32_t a = c.pbase + (uint32_t)row * rowbytes + (uint32_t)(g * B + T * q);
      const uint32_t a4 = on ? (a & ~3u) : kOutOfRange;
      st.ofs[r] = a & 3u;
#pragma unroll
      for (int d = 0; d < PD; ++d)
        st.pk[r][d] = __builtin_amdgcn_raw_buffer_load_b32(c.rp, a4 + 4u * d, 0, 0);
      st.sc[r] = __builtin_amdgcn_raw_buffer_load_b16(
          c.rs, on ? 2u * ((uint32_t)row * (uint32_t)nG + (uint32_t)g) : kOutOfRange, 0, 0);
    }
  };
  // activations of group iteration gi of the cursor's tile (zeros past the
  // tiles, past nG and past the burst)
  auto issue_x = [&](const XCursor &c, int gi, bool live, XStage &st) {
    const int g = g_begin + gi;
    const bool valid = live && c.nrows > 0 && g < nG;
#pragma unroll
    for (int v = 0; v < XL; ++v) {
      const uint32_t o =
          (xoff[v] == kOutOfRange || !valid) ? kOutOfRange : xoff[v] + (uint32_t)(g * G) * 2u;
      if (XW == 4) {
        const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(c.rx, o, 0, 0);
        st.xd[4 * v] = d.x; st.xd[4 * v + 1] = d.y; st.xd[4 * v + 2] = d.z; st.xd[4 * v + 3] = d.w;
      } else {
        const u32x2 d = __builtin_amdgcn_raw_buffer_load_b64(c.rx, o, 0, 0);
        st.xd[2 * v] = d.x; st.xd[2 * v + 1] = d.y;
      }
    }
  };

  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the R x T MFMAs of one group iteration (the A fragments built once for
  // the R MFMA tiles) and the scaled accumulation
  auto compute = [&](const PkStage &sp, const XStage &sx) {
    // A fragments: byte t of the lane's run takes activations 5t .. 5t+4
    u32x4 A[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      auto pair = [&](int e) -> uint32_t {  // (x_e, x_{e+1}) of the run
        return (e & 1) ? __builtin_amdgcn_alignbyte(sx.xd[(e + 1) / 2], sx.xd[(e - 1) / 2], 2u)
                       : sx.xd[e / 2];
      };
      const int e = 5 * t;
      const uint32_t last =
          ((e + 4) & 1) ? (sx.xd[(e + 3) / 2] >> 16) : (sx.xd[(e + 4) / 2] & 0xFFFFu);
      A[t] = u32x4{pair(e), pair(e + 2), last, 0u};
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t w[2];
      w[0] = (__builtin_amdgcn_alignbyte(sp.pk[r][1], sp.pk[r][0], sp.ofs[r]) & wmask[0]) |
             wfill[0];
      w[1] = PD == 3 ? (__builtin_amdgcn_alignbyte(sp.pk[r][PD - 1], sp.pk[r][1], sp.ofs[r]) &
                        wmask[1]) | wfill[1]
                     : 0u;
      u32x4 b[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        // address = byte * 256 + copy * 16: byte (t % 4) of w[t / 4] into byte 1
        const uint32_t sel = 0x0C0C0004u | ((uint32_t)(t & 3) << 8);
        const uint32_t addr = __builtin_amdgcn_perm(copyoff, w[t >> 2], sel);
        b[t] = *(lds_u32x4_c *)(lut_bytes + addr);
      }
      f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < T; ++t)
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[t]),
                                                        __builtin_bit_cast(bf16x8, b[t]), part, 0,
                                                        0, 0);
      const float sc = __half2float(__ushort_as_half((unsigned short)sp.sc[r]));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(sc, part[e], acc[r][e]);
      __builtin_amdgcn_sched_group_barrier(0x100, T, 0);  // table reads
      __builtin_amdgcn_sched_group_barrier(0x008, T, 0);  // MFMAs
    }
  };

  uint32_t flags = 0;
  // end of chunk k: park the partial tiles, add the S parts of each tile in
  // order and store
  auto finish_chunk = [&](int k) {
    const Tile w = tile_of(k);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      red[wv][lane] = acc[r];
      acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      if (part == 0) {
        f32x4 v = red[wv][lane];
        for (int p = 1; p < S; ++p) v += red[wv + p][lane];
        float *__restrict__ y = args.y[w.pi];
        const int row = 16 * r + j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 4 * q + e;
          if (m < M && row < w.nrows) {
            if (v[e] != v[e] && !flags)
              flags = row_has_invalid_byte(
                  args.packed[w.pi] + (int64_t)(w.row0 + row) * rowbytes, rowbytes);
            y[(int64_t)m * ldy + w.row0 + row] = v[e];
          }
        }
      }
      __syncthreads();  // red[] is reused by the next MFMA tile and chunk
    }
  };

  // Chunk by chunk (every wave of the block has the same chunks and group
  // iterations, so the chunk-end barriers are reached together), in bursts
  // of BR group iterations.  A burst issues the activations of its first
  // kXLead iterations, then every packed-byte and scale load of the burst,
  // then streams the activations kXLead iterations ahead.  Loads complete in
  // issue order as far as the wait counter is concerned, so an activation
  // load issued behind a fresh HBM load would wait for it: issuing the
  // burst's HBM loads together leaves one HBM latency per burst and only the
  // activations' cache latency between its iterations.
  //
  // The first burst of the block's first chunk is requested before the
  // decode table is built (the loads fill registers only), so the table
  // build runs under their latency.
  auto issue_burst = [&](const PkCursor &pc, const XCursor &xc, int b0, int nb, XStage (&xs)[kXBuf],
                         PkStage (&st)[BR]) {
#pragma unroll
    for (int d = 0; d < kXLead; ++d) issue_x(xc, b0 + d, d < nb, xs[d]);
#pragma unroll
    for (int i = 0; i < BR; ++i) issue_pk(pc, b0 + i, i < nb, st[i]);
  };
  auto compute_burst = [&](const XCursor &xc, int b0, int nb, XStage (&xs)[kXBuf],
                           PkStage (&st)[BR]) {
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      compute(st[i], xs[i % kXBuf]);
      if (i + kXLead < BR)
        issue_x(xc, b0 + i + kXLead, i + kXLead < nb, xs[(i + kXLead) % kXBuf]);
    }
  };
  // the bursts of chunk k from group iteration b_first on, then its end
  auto chunk_from = [&](int k, const PkCursor &pc, const XCursor &xc, int b_first) {
    for (int b0 = b_first; b0 < ngw; b0 += BR) {
      const int nb = min(BR, ngw - b0);
      XStage xs[kXBuf];
      PkStage st[BR];
      issue_burst(pc, xc, b0, nb, xs, st);
      compute_burst(xc, b0, nb, xs, st);
    }
    finish_chunk(k);
  };
  if (mychunks == 0) return;  // the grid is at most the chunk count: not taken
  {
    PkCursor pc;
    XCursor xc;
    pc.k = 0; set_pk(pc);
    xc.k = 0; set_x(xc);
    {
      const int nb = min(BR, ngw);
      XStage xs[kXBuf];
      PkStage st[BR];
      issue_burst(pc, xc, 0, nb, xs, st);
      // decode table: each thread writes 8 of the 4096 (entry, copy) slots,
      // the copy index rotated by the entry so a wave's writes spread the banks
      {
        const int ent = tid % kLutEntries;
        const uint4 e = lut_entry((uint32_t)ent);
        const int first = (tid / kLutEntries) * (kCopies / 2);
#pragma unroll
        for (int k = 0; k < kCopies / 2; ++k) lut[ent * kCopies + ((first + k + ent) & (kCopies - 1))] = e;
      }
      __syncthreads();
      compute_burst(xc, 0, nb, xs, st);
    }
    chunk_from(0, pc, xc, BR);
  }
  for (int k = 1; k < mychunks; ++k) {
    PkCursor pc;
    XCursor xc;
    pc.k = k; set_pk(pc);
    xc.k = k; set_x(xc);
    chunk_from(k, pc, xc, 0);
  }
  // no load may still be writing this wave's registers when it exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (flags && d_status) atomicOr(d_status, kDevInvalidByte);
}

// Chunk shape: the K split S (TB = 8 / S tiles a chunk).  The smallest S
// whose chunks still fill three quarters of the resident blocks (one per
// CU), so each wave streams the longest runs of groups; every part keeps at
// least one group.
int choose_lgS(int count, int64_t N, int64_t K, int G, int R) {
  const int64_t nG = K / G;
  const int64_t tiles = count * ((N + 16 * R - 1) / (16 * R));
  int lg = 0;
  for (; lg < 3; ++lg) {
    const int64_t tb = kWaves >> lg;
    if ((tiles + tb - 1) / tb >= kMaxBlocks * 3 / 4) break;
    if ((int64_t(1) << (lg + 1)) > nG) break;
  }
  return lg;
}

template <int G, int BR, int R>
void launch_with(const GemvBatch &args, int count, int64_t M, int64_t N, int64_t K, int64_t ldy,
                 int lgS, int32_t *d_status, hipStream_t stream) {
  const int64_t tiles = count * ((N + 16 * R - 1) / (16 * R));
  const int64_t tb = kWaves >> lgS;
  const int nchunks = (int)((tiles + tb - 1) / tb);
  const int grid = nchunks < kMaxBlocks ? nchunks : kMaxBlocks;
  hipLaunchKernelGGL((gemv_kernel<G, BR, R>), dim3(grid), dim3(kThreads), 0, stream, args, count,
                     (int)M, (int)N, (int)K, lgS, nchunks, ldy, d_status);
}

// R MFMA tiles a wave (the activation fragments are built once for them):
// up to 4 from M = 8 rows, 2 from 3, else 1, and no more than leave 192
// chunks (three quarters of the CUs a block) at the largest K split; bursts
// of BR groups, BR * R <= 16.
template <int G>
void launch(const GemvBatch &args, int count, int64_t M, int64_t N, int64_t K, int64_t ldy,
            int32_t *d_status, hipStream_t stream) {
  int R = M >= 8 ? 4 : (M >= 3 ? 2 : 1);
  for (; R > 1; R /= 2) {
    const int lg = choose_lgS(count, N, K, G, R);
    const int64_t tiles = count * ((N + 16 * R - 1) / (16 * R));
    if ((tiles + (kWaves >> lg) - 1) / (kWaves >> lg) >= 192) break;
  }
  const int lgS = choose_lgS(count, N, K, G, R);
  const int64_t ngw = ((K / G) + (1 << lgS) - 1) >> lgS;  // group iterations per chunk
  if (R == 4)
    launch_with<G, 4, 4>(args, count, M, N, K, ldy, lgS, d_status, stream);
  else if (R == 2 && ngw <= 4)
    launch_with<G, 4, 2>(args, count, M, N, K, ldy, lgS, d_status, stream);
  else if (R == 2)
    launch_with<G, 8, 2>(args, count, M, N, K, ldy, lgS, d_status, stream);
  else if (ngw <= 4)
    launch_with<G, 4, 1>(args, count, M, N, K, ldy, lgS, d_status, stream);
  else if (ngw <= 8)
    launch_with<G, 8, 1>(args, count, M, N, K, ldy, lgS, d_status, stream);
  else
    launch_with<G, 16, 1>(args, count, M, N, K, ldy, lgS, d_status, stream);
}

constexpr int64_t kChunkRows = int64_t(1) << 24;  // weight rows per launch

}  // namespace

void launch_gemv(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t M,
                 int64_t N, int64_t K, int G, float *y, int32_t *d_status, hipStream_t stream) {
  if (gemv_m1_supported(M, N, K)) {
    launch_gemv_m1(x, packed, scales, N, K, G, y, d_status, stream);
    return;
  }
  const int64_t rowbytes = (K / G) * bytes_per_group(G);
  for (int64_t n0 = 0; n0 < N; n0 += kChunkRows) {
    const int64_t n = N - n0 < kChunkRows ? N - n0 : kChunkRows;
    GemvBatch args = {};
    args.x[0] = x;
    args.packed[0] = packed + n0 * rowbytes;
    args.scales[0] = scales + n0 * (K / G);
    args.y[0] = y + n0;
    if (G == 64) launch<64>(args, 1, M, n, K, N, d_status, stream);
    else launch<128>(args, 1, M, n, K, N, d_status, stream);
  }
}

void launch_gemv_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                         const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                         int64_t K, int G, int32_t *d_status, hipStream_t stream) {
  if (gemv_m1_supported(M, N, K)) {
    launch_gemv_m1_batched(count, xs, packeds, scales, ys, N, K, G, d_status, stream);
    return;
  }
  if (N > kChunkRows) {
    for (int i = 0; i < count; ++i)
      launch_gemv(xs[i], packeds[i], scales[i], M, N, K, G, ys[i], d_status, stream);
    return;
  }
  for (int i0 = 0; i0 < count; i0 += kMaxBatch) {
    const int cnt = count - i0 < kMaxBatch ? count - i0 : kMaxBatch;
    GemvBatch args = {};
    for (int i = 0; i < cnt; ++i) {
      args.x[i] = xs[i0 + i]; args.packed[i] = packeds[i0 + i];
      args.scales[i] = scales[i0 + i]; args.y[i] = ys[i0 + i];
    }
    if (G == 64) launch<64>(args, cnt, M, N, K, N, d_status, stream);
    else launch<128>(args, cnt, M, N, K, N, d_status, stream);
  }
}

}  // namespace tq
