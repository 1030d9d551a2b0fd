// tq_gemv.hip -- skinny matmul (2 <= M <= 16, and M = 1 for shapes the M = 1
// kernel in tq_gemv_m1.hip does not take) for gfx950.
//
// y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
// (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation":
// the group scale multiplies the group's inner sum; fp32 accumulation.
// "Revisit the Decode Roofline": one-token decode streams every packed weight
// once, so the kernel is bound by HBM bandwidth).
//
// The multiply-adds run on the matrix cores (v_mfma_f32_16x16x32_bf16) with
// one packed byte per lane and MFMA:
//   * The 32 k-slots of an MFMA are four bytes' worth of codes, 8 slots per
//     byte: the byte's five codes and three zeros.  Lane l = j + 16 q feeds
//     byte (T q + t) of the current group of weight row j of a 16-row tile
//     (B operand) and the five matching activations of x row j (A operand;
//     rows j >= M are zero), so after T MFMAs (T = 8 for G=128, 4 for G=64)
//     lane (j, q) holds y[4q + r][row j] partial sums for r = 0..3.
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
// Work: persistent blocks of 8 waves each take a contiguous range of "slabs"
// (16 * TL * 8 / S weight rows of one problem).  Within a slab, wave w covers
// TL (1 or 2) 16-row tiles for one of S consecutive K ranges (S = 1, 2, 4 or 8
// chosen from the shape).  A wave streams the groups of its slabs as one loop
// whose body has no branch around a load, no global store and no barrier, so
// its packed bytes stay four groups in flight across slab boundaries; each
// slab's partial tiles wait in LDS, and every four slabs the S parts of a tile
// are added in a fixed order and stored, so results are deterministic.
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
constexpr int kRing = 4;           // groups of packed bytes in flight per wave
constexpr int kXLead = 2;          // groups of activations in flight per wave
constexpr int kXBuf = 4;           // activation buffers (a divisor of kRing, > kXLead)
constexpr int kSlots = 4;          // slabs per batch whose partial sums wait in LDS

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
  static constexpr int XD = 5 * T / 2;          // activation dwords per lane per group: 20 or 10
  static constexpr int PD = T == 8 ? 3 : 2;     // packed dwords a lane loads per tile and group
};

template <int V>
struct Int {
  static constexpr int value = V;
};

// Grid: persistent blocks over "slabs" of 16 * kTiles * (kWaves / S) weight
// rows of one problem.  S (1, 2, 4, 8) splits K between the waves of a slab;
// a wave covers kTiles (1 or 2) 16-row tiles.
template <int G, int kTiles>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemv_kernel(const GemvBatch args, int count, int M, int N, int K, int lgS, int64_t ldy,
                 int32_t *__restrict__ d_status) {
  using Gm = Geo<G>;
  constexpr int T = Gm::T, XD = Gm::XD, PD = Gm::PD, B = Gm::B;
  __shared__ uint4 lut[kLutEntries * kCopies];
  __shared__ f32x4 res[kSlots][kWaves][kTiles][kWave];

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int nG = K / G;
  const uint32_t rowbytes = (uint32_t)nG * B;
  const int S = 1 << lgS;
  const int part = wv & (S - 1), wtile = wv >> lgS;         // K range and tile pair of the wave
  const int lg_rows = (kTiles == 2 ? 5 : 4) + 3 - lgS;      // slab rows: 16 * kTiles * (kWaves / S)
  const int slab_rows = 1 << lg_rows;
  const int spp = (N + slab_rows - 1) >> lg_rows;           // slabs per problem
  const int nslabs = spp * count;
  const int g_begin = (part * nG) >> lgS, g_end = ((part + 1) * nG) >> lgS;

  // ---- decode table: each thread writes 8 of the 4096 (entry, copy) slots,
  // the copy index rotated by the entry so a wave's writes spread the banks ----
  {
    const int ent = tid % kLutEntries;
    const uint4 e = lut_entry((uint32_t)ent);
    const int first = (tid / kLutEntries) * (kCopies / 2);
#pragma unroll
    for (int k = 0; k < kCopies / 2; ++k) lut[ent * kCopies + ((first + k + ent) & (kCopies - 1))] = e;
  }
  __syncthreads();

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
  // as XD dwords.  Loads are 16 bytes (8 for G=64) at offsets aligned to
  // their size, so with K a multiple of 64 none straddles the end of x; for
  // q = 3 only the first load holds positions < G, the others are made
  // out-of-range (zeros: code positions past G carry no activation).
  constexpr int XL = G == 128 ? 5 : 5;                      // loads per group
  constexpr int XW = G == 128 ? 4 : 2;                      // dwords per load
  uint32_t xoff[XL];
#pragma unroll
  for (int u = 0; u < XL; ++u) {
    const bool on = j < M && !(q == 3 && u >= 1);
    xoff[u] = on ? ((uint32_t)j * (uint32_t)K + (uint32_t)(5 * T * q) + (uint32_t)(XW * 2 * u)) * 2u
                 : kOutOfRange;
  }
  (void)XD;

  uint32_t flags = 0;
  // The block's slabs are the contiguous range [first, first + nmy), taken in
  // batches of up to kSlots.  Within a batch a wave streams its groups
  // [g_begin, g_end) of every slab as one sequence of iterations
  // u = k * ngw + (g - g_begin): the loop body has no branch around a load,
  // no global store and no barrier, so packed bytes stay kRing iterations in
  // flight across slab boundaries.  A slab's per-wave partial sums are parked
  // in LDS; the batch ends with one reduction (fixed order over the S K
  // ranges) and the stores.
  const int ngw = g_end - g_begin;  // >= 1 since S <= nG
  const int per = nslabs / (int)gridDim.x, rem = nslabs - per * (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  const int nmy = per + (bid < rem ? 1 : 0);
  const int first = bid * per + min(bid, rem);

  // Slab cursor: problem pi, slab rs of that problem; stepped without division.
  struct Slab {
    int pi, rs;
  };
  auto step = [&](Slab &c) {
    if (++c.rs == spp) {
      c.rs = 0;
      ++c.pi;
    }
  };
  struct Where {
    int pi, row0, nrows;
  };
  auto where = [&](const Slab &c, bool valid) -> Where {  // not valid: a real problem, no rows
    const int row0 = c.rs << lg_rows;
    return Where{min(c.pi, count - 1), row0, valid ? min(slab_rows, N - row0) : 0};
  };

  struct PkStage {
    uint32_t pk[kTiles][PD];
    uint32_t sc[kTiles];
    uint32_t ofs[kTiles];
  };
  struct XStage {
    uint32_t xd[XL * XW];
  };
  // packed bytes and scales of group g of slab w (rows past w.nrows read 0)
  auto issue_pk = [&](const Where &w, int g, PkStage &st) {
    const uintptr_t pabs =
        reinterpret_cast<uintptr_t>(args.packed[w.pi]) + (uint64_t)w.row0 * rowbytes;
    const uint32_t pbase = (uint32_t)(pabs & 3u);
    // whole dwords: a dword load is fully in range or fully past it (reads 0)
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(reinterpret_cast<const void *>(pabs - pbase),
                  (pbase + (uint32_t)w.nrows * rowbytes + 3u) & ~3u);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(args.scales[w.pi] + (int64_t)w.row0 * nG, (uint32_t)w.nrows * (uint32_t)nG * 2u);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int r = 16 * kTiles * wtile + 16 * t + j;  // slab row of the lane
      const bool on = r < w.nrows;
      const uint32_t a = pbase + (uint32_t)r * rowbytes + (uint32_t)(g * B + T * q);
      const uint32_t a4 = on ? (a & ~3u) : kOutOfRange;
      st.ofs[t] = a & 3u;
#pragma unroll
      for (int d = 0; d < PD; ++d)
        st.pk[t][d] = __builtin_amdgcn_raw_buffer_load_b32(rp, a4 + 4u * d, 0, 0);
      st.sc[t] = __builtin_amdgcn_raw_buffer_load_b16(
          rs, on ? 2u * ((uint32_t)r * (uint32_t)nG + (uint32_t)g) : kOutOfRange, 0, 0);
    }
  };
  // activations of group g of problem pi (all zeros if !valid)
  auto issue_x = [&](bool valid, int pi, int g, XStage &st) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x[pi], (uint32_t)M * (uint32_t)K * 2u);
#pragma unroll
    for (int v = 0; v < XL; ++v) {
      const uint32_t o =
          (xoff[v] == kOutOfRange || !valid) ? kOutOfRange : xoff[v] + (uint32_t)(g * G) * 2u;
      if (XW == 4) {
        const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0);
        st.xd[4 * v] = d.x; st.xd[4 * v + 1] = d.y; st.xd[4 * v + 2] = d.z; st.xd[4 * v + 3] = d.w;
      } else {
        const u32x2 d = __builtin_amdgcn_raw_buffer_load_b64(rx, o, 0, 0);
        st.xd[2 * v] = d.x; st.xd[2 * v + 1] = d.y;
      }
    }
  };

  f32x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the MFMAs of one iteration; all-zero loads add nothing (scale 0)
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
    // all table reads of the iteration first, then the MFMAs
    u32x4 b[kTiles][T];
#pragma unroll
    for (int k = 0; k < kTiles; ++k) {
      uint32_t w[2];
      w[0] = (__builtin_amdgcn_alignbyte(sp.pk[k][1], sp.pk[k][0], sp.ofs[k]) & wmask[0]) | wfill[0];
      w[1] = PD == 3 ? (__builtin_amdgcn_alignbyte(sp.pk[k][PD - 1], sp.pk[k][1], sp.ofs[k]) &
                        wmask[1]) | wfill[1]
                     : 0u;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        // address = byte * 256 + copy * 16: byte (t % 4) of w[t / 4] into byte 1
        const uint32_t sel = 0x0C0C0004u | ((uint32_t)(t & 3) << 8);
        const uint32_t addr = __builtin_amdgcn_perm(copyoff, w[t >> 2], sel);
        b[k][t] = *(lds_u32x4_c *)(lut_bytes + addr);
      }
    }
#pragma unroll
    for (int k = 0; k < kTiles; ++k) {
      f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < T; ++t)
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[t]),
                                                        __builtin_bit_cast(bf16x8, b[k][t]), part, 0, 0, 0);
      const float sc = __half2float(__ushort_as_half((unsigned short)sp.sc[k]));
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[k][r] = fmaf(sc, part[r], acc[k][r]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kTiles * T, 0);  // table reads
    __builtin_amdgcn_sched_group_barrier(0x008, kTiles * T, 0);  // MFMAs
  };

  Slab batch = {first / spp, first - (first / spp) * spp};  // first slab of the batch
  for (int k0 = 0; k0 < nmy; k0 += kSlots) {
    const int nb = min(kSlots, nmy - k0);
    const int U = nb * ngw;
    // issue cursors (slab within the batch, group) for packed bytes and activations
    int pk_k = 0, pk_g = g_begin, x_k = 0, x_g = g_begin;
    Slab pk_c = batch, x_c = batch;
    Where pk_w = where(batch, true), x_w = pk_w;
    auto next_pk = [&]() {
      if (++pk_g == g_end) {
        pk_g = g_begin;
        ++pk_k;
        step(pk_c);
        pk_w = where(pk_c, pk_k < nb);
      }
    };
    auto next_x = [&]() {
      if (++x_g == g_end) {
        x_g = g_begin;
        ++x_k;
        step(x_c);
        x_w = where(x_c, x_k < nb);
      }
    };

    PkStage ring[kRing];
    XStage xs[kXBuf];
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      issue_pk(pk_w, pk_g, ring[d]);
      next_pk();
    }
#pragma unroll
    for (int d = 0; d < kXLead; ++d) {
      issue_x(x_k < nb, x_w.pi, x_g, xs[d]);
      next_x();
    }
    int gi = 0, ks = 0;  // group of the current slab, slab within the batch
    auto round = [&](int u0) {
#pragma unroll
      for (int d = 0; d < kRing; ++d) {
        const int u = u0 + d;
        compute(ring[d], xs[d % kXBuf]);
        issue_pk(pk_w, pk_g, ring[d]);
        next_pk();
        issue_x(x_k < nb, x_w.pi, x_g, xs[(d + kXLead) % kXBuf]);
        next_x();
        if (++gi == ngw && u < U) {  // park the slab's partial sums
#pragma unroll
          for (int t = 0; t < kTiles; ++t) {
            res[ks][wv][t][lane] = acc[t];
            acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          gi = 0;
          ++ks;
        }
      }
    };
    // The first round is peeled so that the loop is entered with its loads
    // in flight in the same order as on its back edge.
    round(0);
    for (int u0 = kRing; u0 < U; u0 += kRing) round(u0);
    __syncthreads();
    if (part == 0) {
      Slab c = batch;
      for (int k = 0; k < nb; ++k, step(c)) {
        const Where w = where(c, true);
        float *__restrict__ y = args.y[w.pi];
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          f32x4 v = res[k][wv][t][lane];
          for (int p = 1; p < S; ++p) v += res[k][wv + p][t][lane];
          const int r = 16 * kTiles * wtile + 16 * t + j;  // slab row of lane column j
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 4 * q + e;
            if (m < M && r < w.nrows) {
              if (v[e] != v[e] && !flags)
                flags = row_has_invalid_byte(
                    args.packed[w.pi] + (int64_t)(w.row0 + r) * rowbytes, rowbytes);
              y[(int64_t)m * ldy + w.row0 + r] = v[e];
            }
          }
        }
      }
    }
    __syncthreads();  // res[] is reused by the next batch
    for (int k = 0; k < nb; ++k) step(batch);
  }
  if (flags && d_status) atomicOr(d_status, kDevInvalidByte);
}

// Slab shape: the K split S and tiles per wave TL.  Prefer two tiles per
// wave (the activation fragments of a group serve both) and the smallest S
// that gives about four slabs per CU; a wave keeps at least one group.
struct Split {
  int S, TL;
};
Split choose_split(int count, int64_t N, int64_t K, int G) {
  const int64_t nG = K / G;
  auto slabs = [&](int S, int TL) {
    const int64_t rows = 16 * TL * (kWaves / S);
    return count * ((N + rows - 1) / rows);
  };
  for (int TL = 2; TL >= 1; --TL)
    for (int S = 1; S <= kWaves; S *= 2) {
      if (S > nG) break;
      if (slabs(S, TL) >= 4 * 256) return Split{S, TL};
    }
  int S = 1;
  while (S * 2 <= kWaves && S * 2 <= nG) S *= 2;
  return Split{S, slabs(S, 2) >= 2 * 256 ? 2 : 1};
}

template <int G>
void launch(const GemvBatch &args, int count, int64_t M, int64_t N, int64_t K, int64_t ldy,
            int32_t *d_status, hipStream_t stream) {
  const Split sp = choose_split(count, N, K, G);
  const int64_t slab_rows = 16 * sp.TL * (kWaves / sp.S);
  const int64_t slabs = count * ((N + slab_rows - 1) / slab_rows);
  const int grid = (int)(slabs < 256 ? slabs : 256);  // one 8-wave block per CU
  if (sp.TL == 2)
    hipLaunchKernelGGL((gemv_kernel<G, 2>), dim3(grid), dim3(kThreads), 0, stream, args, count,
                       (int)M, (int)N, (int)K, __builtin_ctz((unsigned)sp.S), ldy, d_status);
  else
    hipLaunchKernelGGL((gemv_kernel<G, 1>), dim3(grid), dim3(kThreads), 0, stream, args, count,
                       (int)M, (int)N, (int)K, __builtin_ctz((unsigned)sp.S), ldy, d_status);
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
