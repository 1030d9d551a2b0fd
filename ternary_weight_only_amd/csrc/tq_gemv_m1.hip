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
//     so an invalid byte turns the chunk sum into NaN, which is checked once
//     per chunk.  The table is replicated 16 times, copy j living in LDS bank
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

// DPP move restricted to the rows in ROWMASK (other rows read 0).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f32_rows(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROWMASK, 0xF, false));
}

// Sum over each row of 16 lanes; every lane of the row receives the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
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

constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past any range: loads give 0
constexpr int kRing = 4;  // row batches in flight per lane
constexpr int kMaxBatch = 64;  // problems per batched launch

// Up to kMaxBatch same-shaped problems per launch, passed by value.
struct GemvBatch {
  const uint16_t *x[kMaxBatch];
  const uint8_t *packed[kMaxBatch];
  const uint16_t *scales[kMaxBatch];
  float *y[kMaxBatch];
};

// The work of a launch is count * nb row batches (nb per problem); a batch
// is one row per row slot (R = 64W / Lp rows).  Block b takes segment b % S
// of problem b / S: batches [s*nb/S, (s+1)*nb/S), so its activations are
// loaded once.  Threads t = 0..64W-1 map to (row slot rr = t/Lp, chunk
// c = t % Lp); lanes with c >= L idle.  Each lane keeps the packed bytes of
// its next D batches in flight in a register ring; the loop body loads
// unconditionally (batches past the segment read out of range, as zeros) and
// its only store is predicated, so the loads stay D batches ahead.
template <int G, int D, bool WAVE_ROWS>
__global__ __launch_bounds__(kWave * kMaxWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void gemv_m1_kernel(const GemvBatch args, int S, int N, int K, int L, int Lp,
                    int32_t *__restrict__ d_status) {
  __shared__ uint4 lut[kLutEntries * kCopies];
  __shared__ float segsum[2][4 * kMaxWaves];  // R * (Lp/16) = 4W floats per batch

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int R = nthreads / Lp;  // rows per batch
  const int nseg = Lp / 16;     // 16-lane segments per row
  const int rr = tid / Lp;
  const int c = tid % Lp;
  const bool lane_on = c < L;
  const int nG = K / G;
  const uint32_t rowbytes = (uint32_t)L * kChunk;
  const uint32_t total = (uint32_t)N * rowbytes;  // < 2^31, checked by the launcher
  const int gidx = G == 64 ? c : (c >> 1);
  const int nb = (N + R - 1) / R;  // batches per problem
  const int pi = (int)blockIdx.x / S, seg = (int)blockIdx.x - pi * S;
  const int b_begin = (int)(((int64_t)seg * nb) / S), b_end = (int)(((int64_t)(seg + 1) * nb) / S);

  // lane's byte address of batch b is a0 + b * bstep; idle lanes get
  // an offset past any range so their loads read zeros.  Rows past N lie
  // past the end of the buffers and read zeros too (they are never stored).
  const uint32_t a0 = lane_on ? (uint32_t)rr * rowbytes + (uint32_t)c * kChunk : kOutOfRange;
  const uint32_t bstep = (uint32_t)R * rowbytes;
  const uint32_t s0 = lane_on ? 2u * ((uint32_t)rr * (uint32_t)nG + (uint32_t)gidx) : kOutOfRange;
  const uint32_t sstep = 2u * (uint32_t)R * (uint32_t)nG;
  const uint32_t pbytes = (total + 3u) & ~3u, sbytes = (uint32_t)N * (uint32_t)nG * 2u;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(args.packed[pi], pbytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(args.scales[pi], sbytes);
  float *__restrict__ yp = args.y[pi];

  u32x4 ring[D];
  uint32_t rofs[D], rsc[D];
  auto issue = [&](int slot, int b) {  // batches at or past b_end read zeros
    const bool on = b < b_end;
    const uint32_t a = a0 + (uint32_t)b * bstep;
    ring[slot] = __builtin_amdgcn_raw_buffer_load_b128(rp, on ? (a & ~3u) : kOutOfRange, 0, 0);
    rofs[slot] = a & 3u;
    rsc[slot] = __builtin_amdgcn_raw_buffer_load_b16(rs, on ? s0 + (uint32_t)b * sstep : kOutOfRange,
                                                     0, 0);
  };

  // Activations of this lane's chunk as bf16 pairs (x0,x1)(x2,x3)(x4,0) per
  // byte, from x[64c .. 64c+72) (zeros past K and for idle lanes).  The
  // lane's trit p is x[64c + h + p] (h = 1 for the second half of a G=128
  // group); Dn[i] holds the pair (x[64c+h+2i], x[64c+h+2i+1]).
  uint32_t xa[kChunk][3];
  auto load_x = [&](int pi) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x[pi], (uint32_t)K * 2u);
    u32x4 xr[9];
#pragma unroll
    for (int i = 0; i < 9; ++i)
      xr[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, lane_on ? 128u * c + 16u * i : kOutOfRange,
                                                    0, 0);
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
  };
  load_x(pi);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, b_begin + d);

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
  // per-lane byte offset of its table copy, in byte 0 of a perm source
  const uint32_t copyoff = (uint32_t)(tid % kCopies) * 16u;
  __syncthreads();

  lds_bytes_c *lut_bytes = (lds_bytes_c *)(lut);
  uint32_t bad = 0;
  int buf = 0;
  auto round = [&](int g0) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int b = g0 + d;
      // realign the lane's 13 bytes to byte 0
      const uint32_t o = rofs[d];
      const u32x4 A = ring[d];
      const uint32_t aw[4] = {__builtin_amdgcn_alignbyte(A.y, A.x, o),
                              __builtin_amdgcn_alignbyte(A.z, A.y, o),
                              __builtin_amdgcn_alignbyte(A.w, A.z, o),
                              __builtin_amdgcn_alignbyte(0u, A.w, o)};
      const float sc = __half2float(__ushort_as_half((unsigned short)rsc[d]));
      issue(d, b + D);  // refill the slot with the batch D ahead
      u32x4 e[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        // address = byte * 256 + copyoff: byte (j%4) of aw[j/4] into byte 1
        const uint32_t sel = 0x0C0C0004u | ((uint32_t)(j & 3) << 8);
        const uint32_t addr = __builtin_amdgcn_perm(copyoff, aw[j >> 2], sel);
        // one full 128-bit read (ds_read_b128 outruns ds_read_b96 on
        // gfx950); volatile keeps the compiler from narrowing it
        e[j] = *(lds_u32x4_cv *)(lut_bytes + addr);
      }
      float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        float &acc = (j & 3) == 0 ? acc0 : (j & 3) == 1 ? acc1 : (j & 3) == 2 ? acc2 : acc3;
        acc = dot2_bf16(e[j].x, xa[j][0], acc);
        acc = dot2_bf16(e[j].y, xa[j][1], acc);
        acc = dot2_bf16(e[j].z, xa[j][2], acc);
      }
      // The fourth dword of each read is unused; holding it to here stops
      // the register allocator from reusing its register while the read is
      // in flight (that reuse forces a wait right after the read).
#pragma unroll
      for (int j = 0; j < kChunk; ++j) asm volatile("" ::"v"(e[j].w));
      const float pc = (acc0 + acc1) + (acc2 + acc3);
      float part = row16_sum(sc * pc);
      const bool live = b < b_end;
      if (WAVE_ROWS) {
        // a row is Lp <= 64 consecutive lanes of one wave: add its 16-lane
        // rows with row_bcast15/31; the row's last lane holds the sum (an
        // invalid byte anywhere in the row makes it NaN)
        if (Lp >= 32) part += dpp_f32_rows<0x142, 0xA>(part);  // row_bcast:15
        if (Lp >= 64) part += dpp_f32_rows<0x143, 0xC>(part);  // row_bcast:31
        const int n = b * R + rr;
        if (live && c == Lp - 1 && n < N) {
          bad |= (part != part);
          yp[n] = part;
        }
      } else {
        if ((tid & 15) == 0) segsum[buf][rr * nseg + c / 16] = part;
        __syncthreads();
        if (tid < R) {
          const int n = b * R + tid;
          if (live && n < N) {
            float sum = 0.f;
            for (int k = 0; k < nseg; ++k) sum += segsum[buf][tid * nseg + k];
            bad |= (sum != sum);
            yp[n] = sum;
          }
        }
        buf ^= 1;
      }
    }
  };
  // The first round is peeled so that the loop is entered with its loads in
  // flight in the same order as on its back edge.
  if (b_begin < b_end) round(b_begin);
  for (int g0 = b_begin + D; g0 < b_end; g0 += D) round(g0);
  if (bad && d_status) atomicOr(d_status, kDevInvalidByte);
}

// ---------------------------------------------------------------------------
// General fallback: one wave per row, lanes stride over the row's groups.
// Used for 2 <= M <= 16 and for K > 16384.
// ---------------------------------------------------------------------------
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

template <int G>
void launch_m1(const GemvBatch &args, int count, int64_t N, int64_t K, int32_t *d_status,
               hipStream_t stream) {
  const int L = (int)(K / 64);
  const int Lp = 16 * ((L + 15) / 16);
  const int threads = 64 * m1_waves(K);
  const int R = threads / Lp;
  // segments per problem: at most two blocks per CU over the whole launch
  // (two fit the 64 KB table), so every block is resident from the start,
  // and at least one batch per segment
  const int64_t nb = (N + R - 1) / R;
  const int64_t want = count <= 2 * 256 ? (2 * 256) / count : 1;
  const int S = (int)(want < nb ? want : nb);
  const int grid = count * S;
  if (Lp <= 64)
    hipLaunchKernelGGL((gemv_m1_kernel<G, kRing, true>), dim3(grid), dim3(threads), 0, stream,
                       args, S, (int)N, (int)K, L, Lp, d_status);
  else
    hipLaunchKernelGGL((gemv_m1_kernel<G, kRing, false>), dim3(grid), dim3(threads), 0, stream,
                       args, S, (int)N, (int)K, L, Lp, d_status);
}

bool m1_supported(int64_t M, int64_t N, int64_t K) {
  return M == 1 && m1_waves(K) > 0 && N * (K / 64) * 13 < (int64_t(1) << 31);
}

}  // namespace

bool gemv_m1_supported(int64_t M, int64_t N, int64_t K) { return m1_supported(M, N, K); }

void launch_gemv_m1(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t N,
                    int64_t K, int G, float *y, int32_t *d_status, hipStream_t stream) {
  GemvBatch args = {};
  args.x[0] = x; args.packed[0] = packed; args.scales[0] = scales; args.y[0] = y;
  if (G == 64) launch_m1<64>(args, 1, N, K, d_status, stream);
  else launch_m1<128>(args, 1, N, K, d_status, stream);
}

void launch_gemv_m1_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                            const uint16_t *const *scales, float *const *ys, int64_t N, int64_t K,
                            int G, int32_t *d_status, hipStream_t stream) {
  for (int i0 = 0; i0 < count; i0 += kMaxBatch) {
    const int cnt = count - i0 < kMaxBatch ? count - i0 : kMaxBatch;
    GemvBatch args = {};
    for (int i = 0; i < cnt; ++i) {
      args.x[i] = xs[i0 + i]; args.packed[i] = packeds[i0 + i];
      args.scales[i] = scales[i0 + i]; args.y[i] = ys[i0 + i];
    }
    if (G == 64) launch_m1<64>(args, cnt, N, K, d_status, stream);
    else launch_m1<128>(args, cnt, N, K, d_status, stream);
  }
}

}  // namespace tq
