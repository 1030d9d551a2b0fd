// tq_twobit_mm.hip -- matmul over the 2-bit ternary format for any number of
// activation rows and any row length, on the matrix cores (gfx950):
//   y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
// (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation":
// the group scale multiplies the group's inner sum, fp32 accumulation).
// Format (Avenue README, size note: 2-bit packing; "Autoregressive Language
// Model on the 6502 Processor": ternary parameters four a byte): field
// f = c + 1 in two bits, the first weight lowest, G/4 bytes a group, fp16
// group scales; f = 3 is invalid, counts as code 0 and sets the status bit.
//
// Block: 4 waves; wave w computes a BM x 32 tile of y (columns n0 + 32w ..
// n0 + 32w + 31) with v_mfma_f32_16x16x32_bf16 (BM = 16, 32 or 64 rows by
// M).  Groups run through a ring of three: while a group computes, the next
// two load -- the block's BM x G activation tile straight from memory into an
// LDS slot (buffer loads with the lds modifier, XOR-swizzled 16-byte
// chunks), each wave's code bytes and scales into registers.  Per 32-wide k
// step, lane (j, q) of a wave:
//   * looks the two bytes of codes k + 8q .. k + 8q + 7 of W row
//     n0 + 32w + 16t + j (t = 0, 1) up in an LDS table of its four codes as
//     bf16 (exact), giving the B fragment;
//   * reads eight activations x[m][k + 8q ..] of row m0 + 16a + j from the
//     slot (the A fragment; rows past M were loaded as zero);
//   * tests the two bytes for a field of 3 with one bitwise expression.
// At a group's end the fp32 partial tile is scaled by the group's fp16 scale
// and added to the accumulator.  A launch takes up to 64 same-shaped
// problems, one per grid z index.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2_c;
typedef __attribute__((address_space(3))) const unsigned char lds_bytes_c;

constexpr int kThreads = 256;      // 4 waves
constexpr int kTN = 2;             // 16-column MFMA tiles per wave
constexpr int kBN = 4 * 16 * kTN;  // columns per block: 128
constexpr int kCopies = 16;        // table copies; lane l reads copy l % 16
constexpr int kMaxBatch = 64;      // problems per launch
constexpr uint32_t kOutOfRange = 0x80000000u;

struct Mm2Batch {
  const uint16_t *x[kMaxBatch];
  const uint8_t *packed[kMaxBatch];
  const uint16_t *scales[kMaxBatch];
  float *y[kMaxBatch];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// bf16 bits of field f's code c = f - 1 (f = 3, invalid: 0)
__device__ __forceinline__ uint32_t code_bf16(uint32_t f) {
  return f == 0u ? 0xBF80u : (f == 2u ? 0x3F80u : 0u);
}

template <int V>
struct Int {
  static constexpr int value = V;
};

template <int G, int TM>
__global__ __launch_bounds__(kThreads) void matmul2_mfma_kernel(const Mm2Batch args, int M, int N,
                                                                int K, int32_t *d_status) {
  constexpr int BM = 16 * TM;
  constexpr int KS = G / 32;                  // k steps per group
  constexpr int CPR = G / 8;                  // 16-byte chunks of a group's activation row
  // 16-byte LDS loads per thread per group: the tile's BM * CPR chunks, at
  // least one per thread (a small tile's slot is padded: positions past its
  // chunks load zeros and are never read)
  constexpr int XOPS = BM * CPR > kThreads ? BM * CPR / kThreads : 1;
  static_assert(BM * CPR <= kThreads || XOPS * kThreads == BM * CPR,
                "activation tile must split evenly");
  constexpr int SLOT = XOPS * kThreads * 16;  // bytes of one group's activation slot
  constexpr int kDepth = 3;                   // groups in the load ring
  // table: entry of byte b, copy c at byte (b * kCopies + c) * 8: codes of
  // fields 0, 1 in the low dword, 2, 3 in the high dword
  __shared__ __align__(16) u32x2 lut[256 * kCopies];
  __shared__ __align__(16) unsigned char xs_lds[kDepth * SLOT];
  for (int i = threadIdx.x; i < 256 * kCopies; i += kThreads) {
    const uint32_t b = (uint32_t)i / kCopies;
    lut[i] = u32x2{code_bf16(b & 3u) | (code_bf16((b >> 2) & 3u) << 16),
                   code_bf16((b >> 4) & 3u) | (code_bf16((b >> 6) & 3u) << 16)};
  }

  const int pi = (int)blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * kBN + wv * 16 * kTN;
  const int m0 = blockIdx.y * BM;
  const int nG = K / G;
  const uint32_t rb = (uint32_t)K / 4u;  // packed bytes a row
  const uint32_t copyoff = (uint32_t)(lane & (kCopies - 1)) * 8u;
  lds_bytes_c *lut_b = (lds_bytes_c *)lut;

  // rows past M or N lie past the buffers' ranges and read as zero
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x[pi], (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(args.packed[pi], (uint32_t)N * rb);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(args.scales[pi], (uint32_t)N * (uint32_t)nG * 2u);

  // Activation tile of a group: BM rows x G values, loaded straight into LDS
  // by the whole block (op i of thread t fills 16-byte chunk p = 256 i + t of
  // the slot).  Chunk c of row r sits at position c ^ (r % CPR) of its row,
  // so the operand reads (16 rows at one chunk) hit 16 different bank groups.
  uint32_t xg[XOPS];
#pragma unroll
  for (int i = 0; i < XOPS; ++i) {
    const int p = kThreads * i + tid, r = p / CPR, c = (p % CPR) ^ (r % CPR);
    xg[i] = r < BM && m0 + r < M ? ((uint32_t)(m0 + r) * (uint32_t)K + 8u * (uint32_t)c) * 2u
                                 : kOutOfRange;
  }
  const uint32_t wvs = __builtin_amdgcn_readfirstlane(wv);
  auto load_x = [&](int g, int slot) {
#pragma unroll
    for (int i = 0; i < XOPS; ++i) {
      unsigned char *dst = xs_lds + slot * SLOT + 16u * (kThreads * i + 64u * wvs);
      const uint32_t off = xg[i] == kOutOfRange ? kOutOfRange : xg[i] + (uint32_t)(g * G) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void *)dst,
                                               16, off, 0, 0, 0);
    }
  };

  uint32_t poff[kTN], soff[kTN];
#pragma unroll
  for (int t = 0; t < kTN; ++t) {
    const int n = n0 + 16 * t + j;
    poff[t] = n < N ? (uint32_t)n * rb + 2u * (uint32_t)q : kOutOfRange;
    soff[t] = n < N ? (uint32_t)n * (uint32_t)nG * 2u : kOutOfRange;
  }
  // a group's code bytes and scales (registers)
  struct WStage {
    uint32_t wd[KS][kTN];
    uint32_t sc[kTN];
  };
  auto load_w = [&](int g, WStage &w) {
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const uint32_t kk = (uint32_t)(g * G + 32 * s2);
#pragma unroll
      for (int t = 0; t < kTN; ++t)
        w.wd[s2][t] = __builtin_amdgcn_raw_buffer_load_b16(
            rp, poff[t] == kOutOfRange ? kOutOfRange : poff[t] + kk / 4u, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      const uint32_t o = soff[t] == kOutOfRange ? kOutOfRange : soff[t] + 2u * (uint32_t)g;
      w.sc[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, o, 0, 0);
    }
  };
  // loads a group issues: XOPS activation chunks, KS * kTN code halves, kTN scales
  constexpr int kOpsPerGroup = XOPS + KS * kTN + kTN;

  // operand read of row 16 a + j, chunk q + 4 s
  uint32_t aoff[TM][KS];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const int r = 16 * a + j, c = q + 4 * s2;
      aoff[a][s2] = (uint32_t)(r * CPR + (c ^ (r % CPR))) * 16u;
    }

  f32x4 acc[TM][kTN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < kTN; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t bad = 0;

  // group g computes from slot g % 3 and stage w[g % 3] while groups g + 1
  // and g + 2 load into the other two (the ring position is a template
  // argument, so the stages stay in registers)
  WStage w[kDepth];
  load_x(0, 0);
  load_w(0, w[0]);
  load_x(nG > 1 ? 1 : 0, 1);
  load_w(nG > 1 ? 1 : 0, w[1]);
  auto group = [&](auto curc, int g) {
    constexpr int C = decltype(curc)::value, NX = (C + 2) % kDepth;
    // group g + 2's loads (past the last group: a repeat of it, unused)
    const int gn = g + 2 < nG ? g + 2 : nG - 1;
    load_x(gn, NX);
    load_w(gn, w[NX]);
    // this group's loads (issued two groups ago) and the table must be in
    // place; only the next two groups' loads may stay in flight
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kOpsPerGroup)
                 : "memory");
    const unsigned char *xsl = xs_lds + C * SLOT;
    f32x4 part[TM][kTN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int t = 0; t < kTN; ++t) part[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      bf16x8 bq[kTN];
#pragma unroll
      for (int t = 0; t < kTN; ++t) {
        const uint32_t wb = w[C].wd[s2][t] & 0xFFFFu;
        bad |= wb & (wb >> 1) & 0x5555u;  // a field of 3
        const u32x2 e0 = *(lds_u32x2_c *)(lut_b + (((wb & 0xFFu) * kCopies) * 8u + copyoff));
        const u32x2 e1 = *(lds_u32x2_c *)(lut_b + (((wb >> 8) * kCopies) * 8u + copyoff));
        bq[t] = __builtin_bit_cast(bf16x8, u32x4{e0.x, e0.y, e1.x, e1.y});
      }
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const bf16x8 av = *(const __attribute__((address_space(3))) bf16x8 *)(
            (const __attribute__((address_space(3))) unsigned char *)xsl + aoff[a][s2]);
#pragma unroll
        for (int t = 0; t < kTN; ++t)
          part[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[t], part[a][t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      const float sc = __half2float(__ushort_as_half((unsigned short)w[C].sc[t]));
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][t][r] = fmaf(sc, part[a][t][r], acc[a][t][r]);
    }
    // every wave is done with this slot before a later group refills it
    __syncthreads();
  };
  int g = 0;
  for (; g + kDepth <= nG; g += kDepth) {
    group(Int<0>{}, g);
    group(Int<1>{}, g + 1);
    group(Int<2>{}, g + 2);
  }
  if (g < nG) group(Int<0>{}, g);
  if (g + 1 < nG) group(Int<1>{}, g + 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane (j, q) holds rows 4q .. 4q+3 of column j of each 16 x 16 tile; y is
  // written with nontemporal stores (never read back here)
  float *__restrict__ y = args.y[pi];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      const int n = n0 + 16 * t + j;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * a + 4 * q + r;
        if (m < M) __builtin_nontemporal_store(acc[a][t][r], y + (int64_t)m * N + n);
      }
    }
  if (d_status && __builtin_amdgcn_ballot_w64(bad != 0) != 0 && lane == 0)
    atomicOr(d_status, kDevInvalidByte);
}

template <int G, int TM>
void launch_tm(const Mm2Batch &args, int count, int64_t M, int64_t N, int64_t K,
               int32_t *d_status, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + 16 * TM - 1) / (16 * TM)),
                  (unsigned)count);
  hipLaunchKernelGGL((matmul2_mfma_kernel<G, TM>), grid, dim3(kThreads), 0, stream, args,
                     (int)M, (int)N, (int)K, d_status);
}

template <int G>
void launch_g(const Mm2Batch &args, int count, int64_t M, int64_t N, int64_t K,
              int32_t *d_status, hipStream_t stream) {
  if (M <= 16) launch_tm<G, 1>(args, count, M, N, K, d_status, stream);
  else if (M <= 32) launch_tm<G, 2>(args, count, M, N, K, d_status, stream);
  else launch_tm<G, 4>(args, count, M, N, K, d_status, stream);
}

}  // namespace

bool matmul2_supported(int64_t M, int64_t N, int64_t K, int G) {
  // 32-bit buffer offsets: x is M*K*2 bytes, the codes N*K/4, scales N*(K/G)*2
  return (G == 64 || G == 128) && M >= 1 && N >= 1 && K >= G && K % G == 0 &&
         M * K * 2 < (int64_t(1) << 31) && N * (K / 4) < (int64_t(1) << 31) &&
         N * (K / G) * 2 < (int64_t(1) << 31) && (N + kBN) < (int64_t(1) << 30) &&
         M <= int64_t(65535) * 64;  // grid.y <= 65535
}

void launch_matmul2_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                            const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                            int64_t K, int G, int32_t *d_status, hipStream_t stream) {
  // large launches (G = 128, M >= 256, enough 256 x 128 tiles to fill the
  // CUs) go to the persistent kernel of the base-3 matmul, which takes this
  // format too
  if (gemm_wide_supported(count, M, N, K, G)) {
    launch_gemm2_wide(count, xs, packeds, scales, ys, M, N, K, d_status, stream);
    return;
  }
  for (int i0 = 0; i0 < count; i0 += kMaxBatch) {
    const int n = count - i0 < kMaxBatch ? count - i0 : kMaxBatch;
    Mm2Batch args = {};
    for (int i = 0; i < n; ++i) {
      args.x[i] = xs[i0 + i]; args.packed[i] = packeds[i0 + i]; args.scales[i] = scales[i0 + i];
      args.y[i] = ys[i0 + i];
    }
    if (G == 64) launch_g<64>(args, n, M, N, K, d_status, stream);
    else launch_g<128>(args, n, M, N, K, d_status, stream);
  }
}

}  // namespace tq
