// tq_w4a16_gemm.hip -- W4A16 matmul for any number of activation rows on the
// matrix cores (gfx950): y[M,N] = bf16_rne(x[M,K] * W_hat^T), W_hat = q*s + b.
//
// tiny-llm "Week 2 Day 3: Quantize the Model": the stored format
// ("Group-Wise Affine Quantization", "Packed Storage Layout": eight 4-bit
// codes a uint32, the first in the low nibble; a bf16 scale and bias per
// group), the rearranged per-group sum s * sum(x q) + b * sum(x)
// ("Mathematical Formulation") accumulated in fp32 and rounded once to bf16
// ("Computation Flow"), and the dispatch by the number of rows ("GPU
// Dispatch": a matrix-vector schedule for few rows, a matrix schedule above;
// here BM = 16 rows per block for M <= 16, 64 above).
//
// Block: 4 waves; wave w computes a BM x 32 tile of y (columns n0 + 32w ..
// n0 + 32w + 31) with v_mfma_f32_16x16x32_bf16.  A launch takes up to 64
// same-shaped problems, one per grid z index.  Groups run through a ring of
// three: while a group computes, the next two load -- the block's BM x G
// activation tile straight from memory into an LDS slot (buffer loads with
// the lds modifier, XOR-swizzled 16-byte chunks), each wave's codes, scales
// and biases into registers.  Per 32-wide k step, lane (j, q) of a wave:
//   * turns the uint32 of eight codes of W row n0 + 32w + 16t + j at k + 8q
//     (t = 0, 1) into their exact bf16 values (the B fragment: codes 0..15
//     need no rounding);
//   * reads eight activations x[m][k + 8q ..] of row m0 + 16a + j from the
//     slot (the A fragment; rows past M were loaded as zero).
// Per group, one chain of MFMAs gives sum(x q) per (m, n) and a second chain
// against an all-ones B fragment gives sum(x) per m (the bias term's factor,
// in the output layout); at the group's end acc += s * sum(x q) + b * sum(x)
// in fp32.  Products x * q are exact in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int V>
struct Int {
  static constexpr int value = V;
};

constexpr int kThreads = 256;  // 4 waves
constexpr int kTN = 2;         // 16-column MFMA tiles per wave
constexpr int kBN = 4 * 16 * kTN;  // columns per block: 128
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kMaxBatch = 64;  // problems per launch (2.5 KB of kernel arguments)

// Up to kMaxBatch same-shaped problems per launch, passed by value; the
// grid's z index is the problem.
struct W4Batch {
  const uint16_t *x[kMaxBatch];
  const uint32_t *packed[kMaxBatch];
  const uint16_t *scales[kMaxBatch];
  const uint16_t *biases[kMaxBatch];
  uint16_t *y[kMaxBatch];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Eight 4-bit codes (code i in bits 4i..4i+3) -> their bf16 values in k
// order.  Each code becomes an fp32 integer (exact), whose high half is its
// bf16 value; a v_perm joins two high halves.
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  uint32_t p[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float f0 = (float)((lo >> (8 * b)) & 0xFFu);  // code 2b
    const float f1 = (float)((hi >> (8 * b)) & 0xFFu);  // code 2b + 1
    p[b] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8, u32x4{p[0], p[1], p[2], p[3]});
}

template <int G, int TM>
__global__ __launch_bounds__(kThreads) void w4a16_mfma_kernel(const W4Batch args, int M, int N,
                                                              int K) {
  const int pi = (int)blockIdx.z;
  const uint16_t *__restrict__ x = args.x[pi];
  const uint32_t *__restrict__ packed = args.packed[pi];
  const uint16_t *__restrict__ scales = args.scales[pi];
  const uint16_t *__restrict__ biases = args.biases[pi];
  uint16_t *__restrict__ y = args.y[pi];
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
  constexpr int kDepth = 3;  // groups in the load ring: two load while one computes
  __shared__ __align__(16) unsigned char xs_lds[kDepth * SLOT];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * kBN + wv * 16 * kTN;
  const int m0 = blockIdx.y * BM;
  const int nG = K / G;
  const int kw = K / 8;  // code words per row

  // rows past M or N lie past the buffers' ranges and read as zero
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(packed, (uint32_t)N * (uint32_t)kw * 4u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales, (uint32_t)N * (uint32_t)nG * 2u);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(biases, (uint32_t)N * (uint32_t)nG * 2u);

  // Activation tile of a group: BM rows x G values, loaded straight into LDS
  // by the whole block (op i of thread t fills 16-byte chunk p = 256 i + t of
  // the slot).  Chunk c of row r sits at position c ^ (r % CPR) of its row,
  // so the operand reads (16 rows at one chunk) hit 16 different bank groups;
  // the load of position p therefore fetches chunk (p % CPR) ^ (r % CPR).
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
    poff[t] = n < N ? ((uint32_t)n * (uint32_t)kw + (uint32_t)q) * 4u : kOutOfRange;
    soff[t] = n < N ? (uint32_t)n * (uint32_t)nG * 2u : kOutOfRange;
  }
  // a group's codes, scales and biases (registers)
  struct WStage {
    uint32_t wd[KS][kTN];
    uint32_t sc[kTN], bi[kTN];
  };
  auto load_w = [&](int g, WStage &w) {
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const uint32_t kk = (uint32_t)(g * G + 32 * s2);
#pragma unroll
      for (int t = 0; t < kTN; ++t)
        w.wd[s2][t] = __builtin_amdgcn_raw_buffer_load_b32(
            rp, poff[t] == kOutOfRange ? kOutOfRange : poff[t] + (kk / 8u) * 4u, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      const uint32_t o = soff[t] == kOutOfRange ? kOutOfRange : soff[t] + 2u * (uint32_t)g;
      w.sc[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, o, 0, 0);
      w.bi[t] = __builtin_amdgcn_raw_buffer_load_b16(rb, o, 0, 0);
    }
  };
  // loads a group issues: XOPS activation chunks, KS * kTN code words, 2 kTN
  // scale and bias halves
  constexpr int kOpsPerGroup = XOPS + KS * kTN + 2 * kTN;

  const bf16x8 ones = __builtin_bit_cast(
      bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  f32x4 acc[TM][kTN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < kTN; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand read of row 16 a + j, chunk q + 4 s
  uint32_t aoff[TM][KS];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const int r = 16 * a + j, c = q + 4 * s2;
      aoff[a][s2] = (uint32_t)(r * CPR + (c ^ (r % CPR))) * 16u;
    }

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
    // this group's loads (issued two groups ago) must have landed; only the
    // next two groups' may stay in flight
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kOpsPerGroup) : "memory");
    const unsigned char *xsl = xs_lds + C * SLOT;
    float sc[kTN], bi[kTN];
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      sc[t] = bf16_to_f32(w[C].sc[t]);
      bi[t] = bf16_to_f32(w[C].bi[t]);
    }
    f32x4 part[TM][kTN], xs[TM];
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      xs[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kTN; ++t) part[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      bf16x8 bq[kTN];
#pragma unroll
      for (int t = 0; t < kTN; ++t) bq[t] = codes_to_bf16(w[C].wd[s2][t]);
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const bf16x8 av = *(const __attribute__((address_space(3))) bf16x8 *)(
            (const __attribute__((address_space(3))) unsigned char *)xsl + aoff[a][s2]);
#pragma unroll
        for (int t = 0; t < kTN; ++t)
          part[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[t], part[a][t], 0, 0, 0);
        xs[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ones, xs[a], 0, 0, 0);
      }
    }
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int t = 0; t < kTN; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[a][t][r] = fmaf(sc[t], part[a][t][r], fmaf(bi[t], xs[a][r], acc[a][t][r]));
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

  // lane (j, q) holds rows 4q .. 4q+3 of column j of each 16 x 16 tile
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      const int n = n0 + 16 * t + j;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * a + 4 * q + r;
        if (m < M) y[(int64_t)m * N + n] = f32_to_bf16_rne(acc[a][t][r]);
      }
    }
}

template <int G, int TM>
void launch_tm(const W4Batch &args, int count, int64_t M, int64_t N, int64_t K,
               hipStream_t stream) {
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + 16 * TM - 1) / (16 * TM)),
                  (unsigned)count);
  hipLaunchKernelGGL((w4a16_mfma_kernel<G, TM>), grid, dim3(kThreads), 0, stream, args, (int)M,
                     (int)N, (int)K);
}

template <int G>
void launch_g(const W4Batch &args, int count, int64_t M, int64_t N, int64_t K,
              hipStream_t stream) {
  if (M <= 16) launch_tm<G, 1>(args, count, M, N, K, stream);
  else if (M <= 32) launch_tm<G, 2>(args, count, M, N, K, stream);
  else launch_tm<G, 4>(args, count, M, N, K, stream);
}

}  // namespace

bool w4a16_mfma_supported(int64_t M, int64_t N, int64_t K, int G) {
  // 32-bit buffer offsets: x is M*K*2 bytes, the codes N*K/2, scales N*(K/G)*2
  return (G == 64 || G == 128) && M >= 1 && N >= 1 && K >= G && K % G == 0 &&
         M * K * 2 < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31) &&
         (N + kBN) < (int64_t(1) << 30) && M <= int64_t(65535) * 64;  // grid.y <= 65535
}

void launch_w4a16_mfma_batched(int count, const uint16_t *const *xs,
                               const uint32_t *const *packeds, const uint16_t *const *scales,
                               const uint16_t *const *biases, int64_t M, int64_t N, int64_t K,
                               int G, uint16_t *const *ys, hipStream_t stream) {
  for (int i0 = 0; i0 < count; i0 += kMaxBatch) {
    const int n = count - i0 < kMaxBatch ? count - i0 : kMaxBatch;
    W4Batch args = {};
    for (int i = 0; i < n; ++i) {
      args.x[i] = xs[i0 + i]; args.packed[i] = packeds[i0 + i]; args.scales[i] = scales[i0 + i];
      args.biases[i] = biases[i0 + i]; args.y[i] = ys[i0 + i];
    }
    if (G == 64) launch_g<64>(args, n, M, N, K, stream);
    else launch_g<128>(args, n, M, N, K, stream);
  }
}

void launch_w4a16_mfma(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                       const uint16_t *biases, int64_t M, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream) {
  launch_w4a16_mfma_batched(1, &x, &packed, &scales, &biases, M, N, K, G, &y, stream);
}

}  // namespace tq
