// tq_gemv_m1.hip -- decode GEMV for one activation row (M = 1) on gfx950.
//
// y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
// (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation":
// the group scale multiplies the group's inner sum; fp32 accumulation.
// "Revisit the Decode Roofline": one-token decode streams every packed weight
// once, so the kernel is bound by HBM bandwidth).
//
// The kernel (gemv_m1_kernel):
//   * A row's packed bytes are split into 13-byte chunks.  13 bytes hold 65
//     trits: one G=64 group plus its padding trit, or one half of a G=128
//     group (26 bytes), so every chunk belongs to exactly one group and one
//     fp16 scale.  A row has L = K/64 chunks.
//   * Each lane owns one chunk position for all the rows it visits, so its 65
//     activations stay in registers as bf16 pairs (x0,x1)(x2,x3)(x4,0) per
//     byte, with zeros at padding positions.
//   * A byte is decoded by one LDS lookup: a 256-entry table maps it to three
//     bf16 pairs of codes (c0,c1)(c2,c3)(c4,0); v_dot2_f32_bf16 multiplies
//     them with the activation pairs into fp32.  Entries 243..255 hold NaN,
//     so an invalid byte turns its row's sum into NaN.  A NaN row sum can
//     also come from Inf activations or fp32 overflow, so it only marks the
//     row: after the main loop the lanes that stored NaN rows scan those
//     rows' bytes, and only a byte >= 243 sets the invalid-byte status.  The table is replicated 16 times, copy j living in LDS bank
//     group j, and lane l reads copy l%16: the 16 lanes served together hit
//     16 different bank groups whatever the byte values are.
//   * The lookup address (byte * 256 + copy * 16) is built by one v_perm_b32
//     from the data dword and a per-lane constant.
//   * Chunk sums are scaled by the group's fp16 scale, reduced over 16-lane
//     segments with DPP, then across a row's segments through LDS in a fixed
//     order (deterministic results).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const volatile u32x4 lds_u32x4_cv;
typedef __attribute__((address_space(3))) const unsigned char lds_bytes_c;


__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// ---------------------------------------------------------------------------
// M = 1
// ---------------------------------------------------------------------------
constexpr int kCopies = 16;        // LUT replicas, one per 16-byte LDS bank group
constexpr int kLutEntries = 256;   // byte values; 243..255 decode to NaN
constexpr int kChunk = 13;         // bytes per lane chunk
constexpr int kMaxWaves = 8;

// LUT entry for byte value e: three bf16 pairs of the codes of its five
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

// Buffer resource over [p, p + bytes): the hardware range check returns 0 for
// every dword at or past `bytes`, so loads need no branches at the edges.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// 1 if bytes [base, base + len) of the buffer hold a value >= 243 (an
// invalid base-3 byte).  Used only on the rare path of a NaN output; reads
// whole dwords and ignores the bytes outside the range.
__device__ __attribute__((noinline)) uint32_t range_has_invalid_byte(__amdgpu_buffer_rsrc_t r,
                                                                    uint32_t base,
                                                                    uint32_t len) {
  uint32_t hit = 0;
  const uint32_t end = base + len;
  for (uint32_t o = base & ~3u; o < end; o += 4u) {
    const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
#pragma unroll
    for (uint32_t i = 0; i < 4u; ++i) {
      const uint32_t a = o + i;
      if (a >= base && a < end && ((w >> (8u * i)) & 0xFFu) >= 243u) hit = 1u;
    }
  }
  return hit;
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past any range: loads give 0
constexpr int kRing = 4;  // row batches in flight per lane
// Cache policy of the loads of packed weights and their group parameters:
// nontemporal (gfx950's nt bit), since every byte is read once.
constexpr int kStreamed = 2;
constexpr int kMaxBatch = 128;  // problems per launch (6.5 KB of kernel arguments)

// Up to kMaxBatch same-shaped problems per launch, passed by value.
struct GemvBatch {
  const uint16_t *x[kMaxBatch];
  const uint8_t *packed[kMaxBatch];
  const uint16_t *scales[kMaxBatch];
  float *y[kMaxBatch];
};

// Shape of each problem of a launch (problems of one launch may differ in N
// and K): S segments (blocks), the first `rem` of them with q + 1 row
// batches, the others with q.
struct GemvShapes {
  int N[kMaxBatch], K[kMaxBatch], S[kMaxBatch], q[kMaxBatch], rem[kMaxBatch];
};

// The work of a launch is the row batches of its problems (nb per problem);
// a batch is one row per row slot (R = 64W / Lp rows).  Block (s, p) of the
// 2-D grid takes segment s of problem p: batches s, s + S, s + 2S, ... (q or
// q+1 of them), so its activations are loaded once and no block divides,
// and at any moment the blocks of a problem read one contiguous stretch of
// it rather than S stretches far apart.  Problems of one launch may differ in N and K, as long as
// they share the block size and the template configuration.  Threads t = 0..64W-1 map to (row slot rr = t/Lp, chunk
// c = t % Lp); lanes with c >= L idle.  Each lane keeps the packed bytes of
// its next D batches in flight in a register ring; the loop body loads
// unconditionally (batches past the segment read out of range, as zeros) and
// its only store is predicated, so the loads stay D batches ahead.
//
// Start-up order: the activations are requested first, then the first D
// batches of packed bytes; the table is built while both are in flight.
// Then the block stages x once (XL 16-byte pieces per thread at most) in
// LDS, padded by 16 bytes after every 128, and each lane reads its 144-byte
// window from there: lanes 16 apart in chunk index land in different bank
// groups, and the caches see one copy of x per block instead of one per row
// of a batch.  Rows too long for two blocks' LDS per CU (K >= 6848) run one
// block per CU.
template <int G, bool WAVE_ROWS, int XL, bool AL>
__global__ __launch_bounds__(kWave * kMaxWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void gemv_m1_kernel(const GemvBatch args, const GemvShapes shp, int32_t *__restrict__ d_status) {
  __shared__ uint4 lut[kLutEntries * kCopies];
  __shared__ float segsum[2][16 * kMaxWaves];  // 4 batches x R x (Lp/16) = 16W floats
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  extern __shared__ u32x4 xstage_[];  // staged activations (dynamic size)
  lds_u32x4 *xstage = (lds_u32x4 *)xstage_;

  const int pi = (int)blockIdx.y, seg = (int)blockIdx.x;
  if (seg >= shp.S[pi]) return;  // the grid is as wide as the widest problem
  const int N = shp.N[pi], K = shp.K[pi], q = shp.q[pi], rem = shp.rem[pi];
  const int L = K >> 6, Lp = (L + 15) & ~15;
  const float inv_lp = 1.0f / (float)Lp;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int R = (int)(((float)nthreads + 0.5f) * inv_lp);  // rows per batch: nthreads / Lp
  const int nseg = Lp >> 4;  // 16-lane segments per row
  // tid / Lp through a rounded reciprocal: (tid + 1/2) / Lp lies at least
  // 1/(2 Lp) away from an integer, far more than the float error here
  const int rr = (int)(((float)tid + 0.5f) * inv_lp);
  const int c = tid - rr * Lp;
  const bool lane_on = c < L;
  const int nG = K / G;
  const uint32_t rowbytes = (uint32_t)L * kChunk;
  const uint32_t total = (uint32_t)N * rowbytes;  // < 2^30, checked by the launcher
  const int gidx = G == 64 ? c : (c >> 1);
  const int S = shp.S[pi];
  // the segment's batches by local index i in [0, b_end): global batch seg + i*S
  const int b_begin = 0;
  const int b_end = q + (seg < rem ? 1 : 0);

  // activations x[0, K); reads past the end give zeros (the last lane's
  // window reaches 16 bytes beyond x)
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x[pi], (uint32_t)K * 2u);
  const int nxc = (K >> 3) + 1;  // staged 16-byte pieces: x plus one of zeros
  u32x4 xv[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int j = tid + i * nthreads;
    xv[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, j < nxc ? 16u * (uint32_t)j : kOutOfRange,
                                                  0, 0);
  }

  // lane's byte address of local batch b is a0 + b * bstep (its first row is
  // seg*R + rr, S*R rows further per batch); idle lanes get an offset past
  // any range so their loads read zeros.  Rows past N lie past the end of
  // the buffers and read zeros too (they are never stored).
  const uint32_t row0 = (uint32_t)(seg * R + rr);
  const uint32_t a0 = lane_on ? row0 * rowbytes + (uint32_t)c * kChunk : kOutOfRange;
  const uint32_t bstep = (uint32_t)(S * R) * rowbytes;
  const uint32_t s0 = lane_on ? 2u * (row0 * (uint32_t)nG + (uint32_t)gidx) : kOutOfRange;
  const uint32_t sstep = 2u * (uint32_t)(S * R) * (uint32_t)nG;
  const uint32_t pbytes = (total + 3u) & ~3u, sbytes = (uint32_t)N * (uint32_t)nG * 2u;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(args.packed[pi], pbytes);
  // scales are read as the aligned dwords holding them (a 16-bit load's
  // result would be copied between registers at the loop's back edge, which
  // makes the loop wait for every load in flight); the range is widened to
  // whole dwords, which never reaches past a page the buffer touches
  const uintptr_t sp = (uintptr_t)args.scales[pi];
  const uint32_t shead = (uint32_t)(sp & 3u);
  const uint32_t sbytes_al = (sbytes + shead + 3u) & ~3u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc((const void *)(sp - shead), sbytes_al);
  const uint8_t *const pk8 = args.packed[pi];
  const uint8_t *const sc8 = (const uint8_t *)(sp - shead);
  float *__restrict__ yp = args.y[pi];

  // With AL (both batch steps multiples of 4 bytes) a lane's byte offset
  // within its dword and the half holding its scale are the same for every
  // batch, so a batch's loads take the lane's fixed offsets into buffer
  // resources that start b * bstep and b * sstep bytes in (scalar
  // arithmetic; a batch past the segment gets an empty range and reads
  // zeros).
  const uint32_t o_lane = a0 & 3u, sh_lane = ((shead + s0) & 2u) << 3;
  const uint32_t a0al = lane_on ? (a0 & ~3u) : kOutOfRange;
  const uint32_t s0al = lane_on ? ((shead + s0) & ~3u) : kOutOfRange;
  u32x4 ring[kRing];
  uint32_t rsc[kRing];
  auto issue = [&](int slot, int b) {  // batches at or past b_end read zeros
    const bool on = b < b_end;
    if (AL) {
      const int bu = __builtin_amdgcn_readfirstlane(b);  // uniform: keeps this scalar
      const bool onu = bu < b_end;
      const uint32_t pb = (uint32_t)bu * bstep, sb = (uint32_t)bu * sstep;
      const __amdgpu_buffer_rsrc_t rpb = make_rsrc(pk8 + pb, onu ? pbytes - pb : 0u);
      const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sc8 + sb, onu ? sbytes_al - sb : 0u);
      ring[slot] = __builtin_amdgcn_raw_buffer_load_b128(rpb, a0al, 0, kStreamed);
      rsc[slot] = __builtin_amdgcn_raw_buffer_load_b32(rsb, s0al, 0, kStreamed);
    } else {
      const uint32_t a = a0 + (uint32_t)b * bstep;
      ring[slot] = __builtin_amdgcn_raw_buffer_load_b128(rp, on ? (a & ~3u) : kOutOfRange, 0,
                                                         kStreamed);
      rsc[slot] = __builtin_amdgcn_raw_buffer_load_b32(
          rs, on ? ((shead + s0 + (uint32_t)b * sstep) & ~3u) : kOutOfRange, 0, kStreamed);
    }
  };
#pragma unroll
  for (int d = 0; d < kRing; ++d) issue(d, b_begin + d);

  // table: each thread builds one entry and writes a share of its copies;
  // the copy index is rotated by the lane so a wave's 16-byte writes spread
  // over all 16 bank groups
  {
    const int ent = tid % kLutEntries;
    const uint4 e = lut_entry((uint32_t)ent);
    const int per = nthreads >= 2 * kLutEntries ? 2 : 1;  // threads per entry (>= 256 threads)
    const int share = kCopies / per;
    const int first = (tid / kLutEntries) * share;
    if (tid < per * kLutEntries) {
      for (int k = 0; k < share; ++k) {
        const int cp = (first + k + tid) % kCopies;
        lut[ent * kCopies + cp] = e;
      }
    }
  }
  // piece j goes to slot j + j/8
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int j = tid + i * nthreads;
    if (j < nxc) xstage[j + (j >> 3)] = xv[i];
  }
  __syncthreads();

  // Activations of this lane's chunk as bf16 pairs (x0,x1)(x2,x3)(x4,0) per
  // byte, from x[64c .. 64c+72) (pieces 8c .. 8c+8, at slots 9c .. 9c+9 of
  // the staged copy; zeros for idle lanes).  The lane's trit p is
  // x[64c + h + p] (h = 1 for the second half of a G=128 group); Dn[i] holds
  // the pair (x[64c+h+2i], x[64c+h+2i+1]).
  uint32_t xa[kChunk][3];
  {
    u32x4 xr[9];
#pragma unroll
    for (int i = 0; i < 9; ++i)
      xr[i] = lane_on ? xstage[9 * c + i + (i >> 3)] : u32x4{0u, 0u, 0u, 0u};
    const int h = (G == 128) ? (c & 1) : 0;
    uint32_t Dw[36];
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      Dw[4 * i] = xr[i].x; Dw[4 * i + 1] = xr[i].y; Dw[4 * i + 2] = xr[i].z; Dw[4 * i + 3] = xr[i].w;
    }
    uint32_t Dn[34];
#pragma unroll
    for (int i = 0; i < 34; ++i) Dn[i] = __builtin_amdgcn_alignbyte(Dw[i + 1], Dw[i], 2u * h);
    auto pair_at = [&](int p) -> uint32_t {  // (x_p, x_{p+1}) of the lane
      return (p & 1) ? __builtin_amdgcn_alignbyte(Dn[(p + 1) / 2], Dn[(p - 1) / 2], 2u)
                     : Dn[p / 2];
    };
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      xa[j][0] = pair_at(5 * j);
      xa[j][1] = pair_at(5 * j + 2);
      xa[j][2] = pair_at(5 * j + 4) & 0xFFFFu;
    }
    // padding trits carry no activation: p = 64 for G=64 and for the second
    // half of a G=128 group, p = 63 too for the latter
    if (G == 64) {
      xa[kChunk - 1][2] = 0u;
    } else if (h) {
      xa[kChunk - 1][1] &= 0xFFFFu;
      xa[kChunk - 1][2] = 0u;
    }
  }
  // per-lane byte offset of its table copy, in byte 0 of a perm source
  const uint32_t copyoff = (uint32_t)(tid % kCopies) * 16u;

  lds_bytes_c *lut_bytes = (lds_bytes_c *)(lut);
  // bit (round % 32) of nanmask: this lane stored a NaN row in that round
  uint32_t nanmask = 0;
  int buf = 0;
  const int l16 = tid & 15;  // lane within its 16-lane DPP row
  // ds_bpermute byte addresses of the lanes 16 and 32 apart (rows of 32 and
  // 64 lanes add their DPP rows' sums), computed once
  const int bp16 = ((tid & 63) ^ 16) << 2, bp32 = ((tid & 63) ^ 32) << 2;
  const bool hi8 = (l16 & 8) != 0, hi4 = (l16 & 4) != 0;
  // NLIVE: the round's first NLIVE batches lie in the segment; the others
  // (only in a segment's last round) are neither loaded nor computed
  auto round = [&](int g0, auto NLIVE) {
    constexpr int nlive = decltype(NLIVE)::value;
    float v[kRing];
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      if (d >= nlive) {  // resolved at compile time
        v[d] = 0.f;
        continue;
      }
      const int b = g0 + d;
      // realign the lane's 13 bytes to byte 0
      const uint32_t o = AL ? o_lane : ((a0 + (uint32_t)b * bstep) & 3u);
      const u32x4 A = ring[d];
      const uint32_t aw[4] = {__builtin_amdgcn_alignbyte(A.y, A.x, o),
                              __builtin_amdgcn_alignbyte(A.z, A.y, o),
                              __builtin_amdgcn_alignbyte(A.w, A.z, o),
                              __builtin_amdgcn_alignbyte(0u, A.w, o)};
      // the scale is the low or high half of its dword
      const uint32_t sh = AL ? sh_lane : (((shead + s0 + (uint32_t)b * sstep) & 2u) << 3);
      const float sc = __half2float(__ushort_as_half((unsigned short)(rsc[d] >> sh)));
      issue(d, b + kRing);  // refill the slot with the batch kRing ahead
      // the lookups go in two halves (7 + 6 bytes), each read in full
      // before its products, which keeps register use within four waves
      // per SIMD; one accumulator chain per chunk
      float acc = 0.f;
      auto half = [&](auto J0, auto J1) {
        constexpr int j0 = decltype(J0)::value, j1 = decltype(J1)::value;
        u32x4 e[j1 - j0];
#pragma unroll
        for (int j = j0; j < j1; ++j) {
          // address = byte * 256 + copyoff: byte (j%4) of aw[j/4] into byte 1
          const uint32_t sel = 0x0C0C0004u | ((uint32_t)(j & 3) << 8);
          const uint32_t addr = __builtin_amdgcn_perm(copyoff, aw[j >> 2], sel);
          // one full 128-bit read (ds_read_b128 outruns ds_read_b96 on
          // gfx950); volatile keeps the compiler from narrowing it
          e[j - j0] = *(lds_u32x4_cv *)(lut_bytes + addr);
        }
#pragma unroll
        for (int j = j0; j < j1; ++j) {
          acc = dot2_bf16(e[j - j0].x, xa[j][0], acc);
          acc = dot2_bf16(e[j - j0].y, xa[j][1], acc);
          acc = dot2_bf16(e[j - j0].z, xa[j][2], acc);
        }
        // The fourth dword of each read is unused; holding it to here stops
        // the register allocator from reusing its register while the read
        // is in flight (that reuse forces a wait right after the read).
#pragma unroll
        for (int j = j0; j < j1; ++j) asm volatile("" ::"v"(e[j - j0].w));
      };
      half(std::integral_constant<int, 0>{}, std::integral_constant<int, 7>{});
      half(std::integral_constant<int, 7>{}, std::integral_constant<int, kChunk>{});
      v[d] = sc * acc;
    }
    // Sum each batch's chunk values over the 16 lanes of a DPP row, four
    // batches at once: exchange halves across lane bit 3 (row_ror:8), then
    // across bit 2 (row_half_mirror), then add within quads.  Afterwards
    // every lane of quad k (lanes 4k..4k+3 of the row) holds batch k's sum.
    const float keep0 = hi8 ? v[2] : v[0], send0 = hi8 ? v[0] : v[2];
    const float keep1 = hi8 ? v[3] : v[1], send1 = hi8 ? v[1] : v[3];
    const float u0 = keep0 + dpp_f32<0x128>(send0);  // row_ror:8
    const float u1 = keep1 + dpp_f32<0x128>(send1);
    const float keep = hi4 ? u1 : u0, send = hi4 ? u0 : u1;
    float s = keep + dpp_f32<0x141>(send);  // row_half_mirror
    s += dpp_f32<0xB1>(s);                  // quad_perm [1,0,3,2]
    s += dpp_f32<0x4E>(s);                  // quad_perm [2,3,0,1]
    const int k = l16 >> 2;                 // this lane's batch
    if (WAVE_ROWS) {
      // a row is Lp = 16, 32 or 64 lanes of one wave: add its DPP rows
      if (Lp >= 32) s += __int_as_float(__builtin_amdgcn_ds_bpermute(bp16, __float_as_int(s)));
      if (Lp >= 64) s += __int_as_float(__builtin_amdgcn_ds_bpermute(bp32, __float_as_int(s)));
      const int n = (seg + (g0 + k) * S) * R + rr;
      if (c < 16 && (l16 & 3) == 0 && g0 + k < b_end && n < N) {
        nanmask |= (uint32_t)(s != s) << (((g0 - b_begin) >> 2) & 31);
        yp[n] = s;
      }
    } else {
      // rows span waves: add the row's Lp/16 DPP-row sums through LDS
      float *ss = segsum[buf];
      if ((l16 & 3) == 0) ss[(k * R + rr) * nseg + (c >> 4)] = s;
      __syncthreads();
      if (tid < kRing * R) {
        const int kk = tid & 3, r = tid >> 2;
        const int n = (seg + (g0 + kk) * S) * R + r;
        if (g0 + kk < b_end && n < N) {
          float sum = 0.f;
          for (int j = 0; j < nseg; ++j) sum += ss[(kk * R + r) * nseg + j];
          nanmask |= (uint32_t)(sum != sum) << (((g0 - b_begin) >> 2) & 31);
          yp[n] = sum;
        }
      }
      buf ^= 1;
    }
  };
  // The first round is peeled so that the loop is entered with its loads in
  // flight in the same order as on its back edge.  Every segment holds at
  // least one batch (the launcher makes at most nb segments), so the peeled
  // round runs unconditionally: no path reaches the loop around it, with
  // the start-up loads in another order.  A last round with fewer than
  // kRing batches skips the work of the missing ones.
  const std::integral_constant<int, kRing> full{};
  round(b_begin, full);
  int g0 = b_begin + kRing;
  for (; g0 + kRing < b_end; g0 += kRing) round(g0, full);
  if (g0 < b_end) {
    if (b_end - g0 <= 2) round(g0, std::integral_constant<int, 2>{}); else round(g0, full);
  }
  if (nanmask && d_status) {
    // Rare path: scan the rows this lane stored in rounds whose mask bit is
    // set (rounds 32 apart share a bit, so some rows may be scanned for
    // nothing) for a byte >= 243.
    const int k = WAVE_ROWS ? (l16 >> 2) : (tid & 3);
    const int r = WAVE_ROWS ? rr : (tid >> 2);
    uint32_t hit = 0;
    for (int g0 = b_begin; g0 < b_end && !hit; g0 += kRing) {
      const int n = (seg + (g0 + k) * S) * R + r;
      if (((nanmask >> (((g0 - b_begin) >> 2) & 31)) & 1u) && g0 + k < b_end && n < N)
        hit = range_has_invalid_byte(rp, (uint32_t)n * rowbytes, rowbytes);
    }
    if (hit) atomicOr(d_status, kDevInvalidByte);
  }
}

// Blocks of W waves whose threads tile whole rows: Lp = 16*ceil(K/1024)
// lanes per row must divide 64*W with W <= 8; 0 when no such W exists.
int m1_waves(int64_t K) {
  if (K % 64 != 0 || K / 64 > 256) return 0;
  const int L = (int)(K / 64);
  const int s = (L + 15) / 16;
  int g4 = 1;
  for (int d = 1; d <= 4; ++d)
    if (s % d == 0 && 4 % d == 0) g4 = d;
  const int w0 = s / g4;  // smallest W with 64W % Lp == 0
  if (w0 > 8) return 0;
  return w0 * (8 / w0);   // up to 8 waves per block
}

// LDS of one block: the table, the segment sums and the staged activations
// (16-byte pieces of x plus a zero piece, one pad slot after every 8);
// two blocks per CU need at most half of the CU's 160 KB
constexpr int kStaticLds = kLutEntries * kCopies * 16 + 2 * 16 * kMaxWaves * 4;
int m1_stage_bytes(int K) {
  const int nxc = K / 8 + 1;
  return 16 * (nxc + (nxc - 1) / 8 + 1);
}
bool m1_staged(int K) { return kStaticLds + m1_stage_bytes(K) <= 80 * 1024; }
// Longer rows stage x too, with one block per CU (the whole 160 KB): a block
// then reads x once from the caches instead of each lane its own window.
bool m1_staged_one(int K) { return kStaticLds + m1_stage_bytes(K) <= 160 * 1024; }
constexpr int kXlOne = 5;  // staged pieces per thread when one block holds a CU (K <= 16384)

// Segments of a problem with nb row batches whose share of a launch is
// `share` blocks out of `slots` (512: two blocks per CU -- two fit the 64 KB
// table; 256 when a block's staged activations take a CU's LDS -- so every
// block is resident from the start).  A block runs whole rounds of kRing
// batches (a round's batches past its segment are computed on zeros), so a
// CU's work is about ceil(blocks / per-CU) blocks times the rounds of the
// longest segment, the launch counting slots / share problems like this
// one.  Among the segment counts up to the share that give each
// segment a batch, take the one with the least work on the busiest CU, then
// the least work in all, then the most blocks (more loads in flight).
int m1_segments(int64_t share, int64_t nb, int64_t slots) {
  const int64_t count = share >= slots ? 1 : slots / share;
  int64_t smax = share < nb ? share : nb;
  int best = 1;
  int64_t best_cu = -1, best_all = -1;
  for (int64_t S = 1; S <= smax; ++S) {
    const int64_t q = nb / S, rem = nb % S;
    const int64_t rounds_long = (q + (rem ? 1 : 0) + kRing - 1) / kRing;
    const int64_t rounds_short = (q + kRing - 1) / kRing;
    const int64_t blocks = (int64_t)count * S;
    const int64_t cu = ((blocks + slots - 1) / slots) * rounds_long;
    const int64_t all = (int64_t)count * (rem * rounds_long + (S - rem) * rounds_short);
    if (best_cu < 0 || cu < best_cu || (cu == best_cu && all <= best_all)) {
      best = (int)S;
      best_cu = cu;
      best_all = all;
    }
  }
  return best;
}

// Launch configuration of one problem: the block size and the kernel's
// template parameters.  Problems with equal configurations share launches.
struct M1Config {
  int threads;
  bool wave_rows;  // rows of 16, 32 or 64 lanes, inside one wave
  bool one_per_cu; // staged activations too large for two blocks per CU
  int xl;          // staged pieces per thread: 1, 2, 3 or kXlOne
  bool aligned;    // both batch steps in whole dwords
  bool operator==(const M1Config &o) const {
    return threads == o.threads && wave_rows == o.wave_rows && one_per_cu == o.one_per_cu &&
           xl == o.xl && aligned == o.aligned;
  }
};

M1Config m1_config(int64_t K, int G) {
  M1Config c;
  const int L = (int)(K / 64), Lp = 16 * ((L + 15) / 16);
  c.threads = 64 * m1_waves(K);
  const int R = c.threads / Lp;
  c.wave_rows = Lp == 16 || Lp == 32 || Lp == 64;
  const int xl = ((int)(K >> 3) + 1 + c.threads - 1) / c.threads;
  // rows of K >= 6848 (two blocks' LDS per CU exceeded) take 112 to 256
  // lanes, which span waves, and at most kXlOne pieces a thread
  c.one_per_cu = !m1_staged((int)K);
  c.xl = c.one_per_cu ? kXlOne : (xl <= 1 ? 1 : (xl <= 2 ? 2 : 3));
  const int64_t bstep = (int64_t)R * L * kChunk, sstep = 2 * (int64_t)R * (K / G);
  c.aligned = bstep % 4 == 0 && sstep % 4 == 0;
  return c;
}

template <int G, bool WR, int XL, bool AL>
void launch_m1_k(const GemvBatch &args, const GemvShapes &shp, dim3 grid, int threads, int lds,
                 int32_t *d_status, hipStream_t stream) {
  if (kStaticLds + lds > 64 * 1024) {
    // a block above 64 KB of LDS (one per CU): allow the dynamic part
    static const hipError_t set = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemv_m1_kernel<G, WR, XL, AL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - kStaticLds);
    (void)set;
  }
  hipLaunchKernelGGL((gemv_m1_kernel<G, WR, XL, AL>), grid, dim3(threads), lds, stream, args,
                     shp, d_status);
}

template <int G, bool WR, int XL>
void launch_m1_al(const M1Config &c, const GemvBatch &args, const GemvShapes &shp, dim3 grid,
                  int lds, int32_t *d_status, hipStream_t stream) {
  if (c.aligned)
    launch_m1_k<G, WR, XL, true>(args, shp, grid, c.threads, lds, d_status, stream);
  else
    launch_m1_k<G, WR, XL, false>(args, shp, grid, c.threads, lds, d_status, stream);
}

template <int G, bool WR>
void launch_m1_wr(const M1Config &c, const GemvBatch &args, const GemvShapes &shp, dim3 grid,
                  int lds, int32_t *d_status, hipStream_t stream) {
  if constexpr (!WR) {
    if (c.one_per_cu) {  // only rows that span waves are this long
      launch_m1_al<G, WR, kXlOne>(c, args, shp, grid, lds, d_status, stream);
      return;
    }
  }
  if (c.xl == 1)
    launch_m1_al<G, WR, 1>(c, args, shp, grid, lds, d_status, stream);
  else if (c.xl == 2)
    launch_m1_al<G, WR, 2>(c, args, shp, grid, lds, d_status, stream);
  else
    launch_m1_al<G, WR, 3>(c, args, shp, grid, lds, d_status, stream);
}

// One launch over up to kMaxBatch problems that share configuration c.
template <int G>
void launch_m1(const M1Config &c, int count, const uint16_t *const *xs,
               const uint8_t *const *packeds, const uint16_t *const *scales, float *const *ys,
               const int64_t *Ns, const int64_t *Ks, int32_t *d_status, hipStream_t stream) {
  GemvBatch args = {};
  GemvShapes shp = {};
  int smax = 1, lds = 0;
  // the blocks of a launch (512, or 256 at one per CU) are shared out in
  // proportion to the problems' sizes (weights, i.e. packed bytes)
  const int slots = c.one_per_cu ? 256 : 512;
  double total = 0.0;
  for (int i = 0; i < count; ++i) total += (double)Ns[i] * (double)Ks[i];
  int segs[kMaxBatch], most[kMaxBatch], order[kMaxBatch];
  for (int i = 0; i < count; ++i) {
    const int L = (int)(Ks[i] / 64), Lp = 16 * ((L + 15) / 16), R = c.threads / Lp;
    const int64_t nb = (Ns[i] + R - 1) / R;
    int64_t share = (int64_t)((double)slots * ((double)Ns[i] * (double)Ks[i]) / total);
    if (share < 1) share = 1;
    segs[i] = m1_segments(share, nb, slots);
    most[i] = (int)((nb + segs[i] - 1) / segs[i]);  // batches of the longest segment
    order[i] = i;
  }
  // Problems with the longest segments first: blocks are dispatched in
  // order, one to each CU before any CU gets a second, so the heaviest
  // blocks share their CUs with lighter ones.
  std::stable_sort(order, order + count, [&](int a, int b) { return most[a] > most[b]; });
  for (int j = 0; j < count; ++j) {
    const int i = order[j];
    args.x[j] = xs[i]; args.packed[j] = packeds[i]; args.scales[j] = scales[i]; args.y[j] = ys[i];
    const int L = (int)(Ks[i] / 64), Lp = 16 * ((L + 15) / 16), R = c.threads / Lp;
    const int64_t nb = (Ns[i] + R - 1) / R;
    const int S = segs[i];
    shp.N[j] = (int)Ns[i];
    shp.K[j] = (int)Ks[i];
    shp.S[j] = S;
    shp.q[j] = (int)(nb / S);
    shp.rem[j] = (int)(nb % S);
    if (S > smax) smax = S;
    if (m1_stage_bytes((int)Ks[i]) > lds) lds = m1_stage_bytes((int)Ks[i]);
  }
  const dim3 grid(smax, count);
  if (c.wave_rows)
    launch_m1_wr<G, true>(c, args, shp, grid, lds, d_status, stream);
  else
    launch_m1_wr<G, false>(c, args, shp, grid, lds, d_status, stream);
}

bool m1_supported(int64_t M, int64_t N, int64_t K) {
  // packed bytes below 1 GiB: 32-bit offsets never wrap; the staged
  // activations fit a configuration (always so for the K that m1_waves takes)
  if (M != 1 || m1_waves(K) <= 0 || N * (K / 64) * 13 >= (int64_t(1) << 30)) return false;
  const M1Config c = m1_config(K, 128);
  const int xl = ((int)(K >> 3) + 1 + c.threads - 1) / c.threads;
  return c.one_per_cu ? (!c.wave_rows && m1_staged_one((int)K) && xl <= kXlOne) : xl <= 3;
}

}  // namespace

bool gemv_m1_supported(int64_t M, int64_t N, int64_t K) { return m1_supported(M, N, K); }

void launch_gemv_m1_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                            const uint16_t *const *scales, float *const *ys, const int64_t *Ns,
                            const int64_t *Ks, int G, int32_t *d_status, hipStream_t stream) {
  // problems in order, grouped by configuration, up to kMaxBatch per launch
  const uint16_t *gx[kMaxBatch];
  const uint8_t *gp[kMaxBatch];
  const uint16_t *gs[kMaxBatch];
  float *gy[kMaxBatch];
  int64_t gn[kMaxBatch], gk[kMaxBatch];
  std::vector<unsigned char> done((size_t)(count > 0 ? count : 0), 0);
  for (int i0 = 0; i0 < count; ++i0) {
    if (done[i0]) continue;
    const M1Config c = m1_config(Ks[i0], G);
    int n = 0;
    for (int i = i0; i < count; ++i) {
      if (done[i] || !(m1_config(Ks[i], G) == c)) continue;
      done[i] = true;
      gx[n] = xs[i]; gp[n] = packeds[i]; gs[n] = scales[i]; gy[n] = ys[i];
      gn[n] = Ns[i]; gk[n] = Ks[i];
      if (++n == kMaxBatch) {
        if (G == 64) launch_m1<64>(c, n, gx, gp, gs, gy, gn, gk, d_status, stream);
        else launch_m1<128>(c, n, gx, gp, gs, gy, gn, gk, d_status, stream);
        n = 0;
      }
    }
    if (n > 0) {
      if (G == 64) launch_m1<64>(c, n, gx, gp, gs, gy, gn, gk, d_status, stream);
      else launch_m1<128>(c, n, gx, gp, gs, gy, gn, gk, d_status, stream);
    }
  }
}

void launch_gemv_m1(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t N,
                    int64_t K, int G, float *y, int32_t *d_status, hipStream_t stream) {
  launch_gemv_m1_grouped(1, &x, &packed, &scales, &y, &N, &K, G, d_status, stream);
}

void launch_gemv_m1_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                            const uint16_t *const *scales, float *const *ys, int64_t N, int64_t K,
                            int G, int32_t *d_status, hipStream_t stream) {
  for (int i0 = 0; i0 < count; i0 += kMaxBatch) {
    const int cnt = count - i0 < kMaxBatch ? count - i0 : kMaxBatch;
    int64_t ns[kMaxBatch], ks[kMaxBatch];
    for (int i = 0; i < cnt; ++i) { ns[i] = N; ks[i] = K; }
    launch_gemv_m1_grouped(cnt, xs + i0, packeds + i0, scales + i0, ys + i0, ns, ks, G, d_status,
                           stream);
  }
}

}  // namespace tq
