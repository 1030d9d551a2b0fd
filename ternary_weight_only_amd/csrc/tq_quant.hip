// tq_quant.hip -- quantize/pack and unpack kernels for gfx950.
//
// Format: precisit "pack-unpack-run" README, codec.py description and
// scale-rule paragraph: per group of G weights an fp16 scale equal to the
// mean of |w| (one round-half-even from the exact sum), codes c = sign(w)
// where |w| > s/2 (ties to 0), five base-3 digits (c + 1) per byte with the
// first weight least significant, ceil(G/5) bytes per group, padding trits of
// code 0, byte values 243..255 invalid.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tq_digits.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxBlocks = 16384;  // blocks of one launch, over all its problems

// ---------------------------------------------------------------------------
// fp16 rounding of a fixed-point magnitude.
//
// A bf16 magnitude u (sign cleared) is sig * 2^(e - 133) with sig <= 255:
// normal E = u >> 7 >= 1 gives sig = 128 + (u & 127), e = E - 1; subnormal
// E = 0 gives sig = u & 127, e = 0.  A group's magnitudes are summed as
// integers sig << (e - e_max + kWin), exact while every shift is >= 0.
// ---------------------------------------------------------------------------
constexpr int kWin = 48;  // 128 terms of 255 << 48 stay below 2^63

// Round-half-even of T / 2^r to an integer (r >= 1; T < 2^63).
__device__ __forceinline__ uint64_t rne_shift(uint64_t T, uint32_t r) {
  if (r >= 64) return 0;
  const uint64_t q = T >> r;
  const uint64_t rem = T & ((1ull << r) - 1);
  const uint64_t half = 1ull << (r - 1);
  return q + ((rem > half) || (rem == half && (q & 1)) ? 1 : 0);
}

// fp16 bits of RNE(T * 2^sh * 2^-24), i.e. the value T * 2^sh in units of the
// fp16 subnormal step.  Sets *ovf and returns 0x7C00 when it rounds to >= 65520.
__device__ __forceinline__ uint32_t f16_bits_of_fixed(uint64_t T, int sh, bool *ovf) {
  *ovf = false;
  if (T == 0) return 0;
  if (sh >= 0) { *ovf = true; return 0x7C00; }  // T >= 2^55 here: far beyond 65504
  const int r = -sh;
  const int L = 63 - __clzll((long long)T);
  if (L < r + 10) return (uint32_t)rne_shift(T, (uint32_t)r);  // below 1024 steps
  const int k = L - r - 10;                                    // value in [2^(10+k), 2^(11+k))
  if (k >= 30) { *ovf = true; return 0x7C00; }
  const uint32_t bits = ((uint32_t)k << 10) + (uint32_t)rne_shift(T, (uint32_t)(L - 10));
  if (bits >= 0x7C00) { *ovf = true; return 0x7C00; }
  return bits;
}

// Exact fallback for one group: 320-bit sum of sig << e, then one rounding of
// sum * 2^-133 / 2^t to fp16.  Only runs for groups whose fixed-point window
// dropped bits that could change the rounding.
__device__ __noinline__ uint32_t f16_scale_exact(const uint16_t *grp, int G, int t, bool *ovf) {
  uint64_t A[5] = {0, 0, 0, 0, 0};
  for (int j = 0; j < G; ++j) {
    const uint32_t u = grp[j] & 0x7FFFu;
    const uint32_t E = u >> 7, m = u & 0x7Fu;
    const uint64_t sig = E ? 128u + m : m;
    const int e = E ? (int)E - 1 : 0;
    const int limb = e >> 6, off = e & 63;
    const uint64_t lo = sig << off;
    const uint64_t hi = off ? (sig >> (64 - off)) : 0;
    uint64_t carry = 0;
    for (int i = limb; i < 5; ++i) {
      const uint64_t add = (i == limb) ? lo : (i == limb + 1 ? hi : 0);
      const uint64_t s1 = A[i] + add;
      const uint64_t c1 = s1 < add;
      const uint64_t s2 = s1 + carry;
      carry = c1 + (s2 < s1);
      A[i] = s2;
    }
  }
  int L = -1;
  for (int i = 4; i >= 0 && L < 0; --i)
    if (A[i]) L = 64 * i + 63 - __clzll((long long)A[i]);
  *ovf = false;
  if (L < 0) return 0;
  // value in units of 2^-24: A / 2^(109 + t)
  const int r = 109 + t;
  auto bits_at = [&](int pos, int n) -> uint64_t {  // bits [pos, pos+n), n <= 32
    uint64_t v = 0;
    for (int b = 0; b < n; ++b) {
      const int p = pos + b;
      if (p >= 0 && p < 320) v |= ((A[p >> 6] >> (p & 63)) & 1ull) << b;
    }
    return v;
  };
  auto any_below = [&](int pos) -> bool {
    for (int p = 0; p < pos && p < 320; ++p)
      if ((A[p >> 6] >> (p & 63)) & 1ull) return true;
    return false;
  };
  auto rne_at = [&](int d) -> uint64_t {  // RNE(A / 2^d), result < 2^13
    const uint64_t q = bits_at(d, 13);
    const bool half = bits_at(d - 1, 1) != 0;
    const bool sticky = any_below(d - 1);
    return q + ((half && (sticky || (q & 1))) ? 1 : 0);
  };
  if (L < r + 10) return (uint32_t)rne_at(r);
  const int k = L - r - 10;
  if (k >= 30) { *ovf = true; return 0x7C00; }
  const uint32_t bits = ((uint32_t)k << 10) + (uint32_t)rne_at(L - 10);
  if (bits >= 0x7C00) { *ovf = true; return 0x7C00; }
  return bits;
}

// bf16 bits of the fp16 value h (finite, non-negative here): fp16 -> fp32 is
// exact, then one round to nearest, ties to even, to 8 significant bits.
__device__ __forceinline__ uint32_t bf16_of_f16(uint32_t h) {
  const uint32_t u = __float_as_uint(__half2float(__ushort_as_half((unsigned short)h)));
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Lane i's partner in butterfly step k of a 16-lane group, as a DPP move:
// i^1, i^2 (quad permutes), then 7-i within each 8 lanes (row_half_mirror)
// and 15-i within 16 (row_mirror).  Every step pairs lanes symmetrically, so
// a commutative reduction leaves the same value in all lanes of the group.
template <int STEP>
__device__ __forceinline__ uint32_t dpp_partner(uint32_t v) {
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, kWave);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = shfl_xor_u32((uint32_t)v, mask);
  const uint32_t hi = shfl_xor_u32((uint32_t)(v >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// quantize + pack.
// A wave handles a chunk of 2048 consecutive weights (= 2048/G whole groups,
// since the flat group index n*(K/G) + g addresses w at (n*(K/G) + g) * G).
// Each lane loads 32 bf16 with four 128-bit loads; G/32 lanes (4 or 2) share
// a group and combine their sums, maxima and flags with DPP moves and xor
// shuffles.  Magnitudes and codes are worked two weights a dword with packed
// 16-bit integer operations; digits d = c + 1 are held one a byte.
//
// MODE kPack3: bytes of five base-3 digits, each formed by the lane whose
// digits it starts in (a dot product of four digit bytes with 1, 3, 9, 27
// plus 81 times the fifth).  kPack2: four 2-bit fields a byte.  The QAT
// forward (w_hat = bf16(c * s)) is fake_quantize_kernel below.
// ---------------------------------------------------------------------------
// Problems of one launch (blockIdx.y picks one), all of one shape.
struct QuantBatch {
  const uint16_t *w[kQuantMaxBatch];
  uint8_t *packed[kQuantMaxBatch];
  uint16_t *scales[kQuantMaxBatch];
  uint16_t *w_hat[kQuantMaxBatch];
};

constexpr int kWPL = 32;             // weights per lane
constexpr int kChunk = kWave * kWPL;  // weights per wave and chunk

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Nontemporal loads and stores, for data used once where each instruction
// covers whole cache lines (a wave's 16-byte accesses contiguous).  The
// quantize kernel's weight loads stay cached: each of its four loads reads a
// quarter of the same lines, and nontemporal loads there fetched them again.
__device__ __forceinline__ uint4 load_streamed(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_streamed(void *p, uint32_t a, uint32_t b, uint32_t c,
                                               uint32_t d) {
  __builtin_nontemporal_store(u32x4{a, b, c, d}, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// MODE: kPack3 (base-3 bytes), kPack2 (2-bit fields).
constexpr int kPack3 = 0, kPack2 = 2;

template <int G, int MODE>
__global__ __launch_bounds__(kBlock) void quantize_pack_kernel(const QuantBatch args,
                                                               int64_t total_groups,
                                                               int32_t *__restrict__ d_status) {
  const uint16_t *__restrict__ w = args.w[blockIdx.y];
  uint8_t *__restrict__ packed = args.packed[blockIdx.y];
  uint16_t *__restrict__ scales = args.scales[blockIdx.y];
  constexpr int LPG = G / kWPL;            // lanes per group: 4 or 2
  constexpr int GPC = kChunk / G;          // groups per chunk
  constexpr int B = bytes_per_group(G);    // bytes per group
  constexpr int LOG2G = (G == 64) ? 6 : 7;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane % LPG;
  const int qg = lane / LPG;
  const int64_t nchunks = (total_groups + GPC - 1) / GPC;

  // the next chunk's weights are loaded before this chunk's work
  const int64_t bstep = (int64_t)gridDim.x * kWavesPerBlock;
  uint32_t nraw[16];
  auto load_chunk = [&](int64_t base) {
    const int64_t chunk = base + wv;
    const int64_t gi = chunk * GPC + qg;
    const bool on = chunk < nchunks && gi < total_groups;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (on) v = reinterpret_cast<const uint4 *>(w + gi * G + sub * kWPL)[i];
      nraw[4 * i] = v.x; nraw[4 * i + 1] = v.y; nraw[4 * i + 2] = v.z; nraw[4 * i + 3] = v.w;
    }
  };
  load_chunk((int64_t)blockIdx.x * kWavesPerBlock);
  for (int64_t base = (int64_t)blockIdx.x * kWavesPerBlock; base < nchunks; base += bstep) {
    const int64_t chunk = base + wv;
    const int64_t gi = chunk * GPC + qg;
    const bool active = chunk < nchunks && gi < total_groups;

    uint32_t raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = nraw[i];
    if (base + bstep < nchunks) load_chunk(base + bstep);
    // magnitudes, two a dword (sign bits cleared)
    uint32_t m2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) m2[i] = raw[i] & 0x7FFF7FFFu;

    // Fast path.  The sum of |w| in fp32: each lane adds its 32 magnitudes in
    // a fixed tree (depth 5), then an xor butterfly over the group's LPG lanes
    // (fp32 addition commutes, so every lane ends with the same sum S_hat).
    // Along any path there are at most 5 + log2(LPG) <= 7 rounded additions
    // of non-negative terms, so |S_hat - S| <= 7 * 2^-24 * S, plus at most
    // G * 2^-126 should subnormals be flushed.  With E = 2^-19 S_hat + 2^-118
    // the exact sum lies in [S_hat - E, S_hat + E] even after the rounding of
    // those two operations; when both ends, divided by G, round to the same
    // fp16 value, so does the exact mean (rounding is monotonic).  Otherwise
    // the group takes the exact path below.
    float f[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f[2 * i] = __uint_as_float(m2[i] << 16);
      f[2 * i + 1] = __uint_as_float(m2[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int st = 1; st < 32; st <<= 1)
#pragma unroll
      for (int i = 0; i < 32; i += 2 * st) f[i] += f[i + st];
    float acc = f[0];
    u16x2 mx = as_u16x2(m2[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = __builtin_elementwise_max(mx, as_u16x2(m2[i]));
    uint32_t maxmag = mx.x > mx.y ? mx.x : mx.y;
    auto step = [&](auto k) {
      acc += __uint_as_float(dpp_partner<decltype(k)::value>(__float_as_uint(acc)));
      const uint32_t o = dpp_partner<decltype(k)::value>(maxmag);
      maxmag = o > maxmag ? o : maxmag;
    };
    step(std::integral_constant<int, 0>{});
    if constexpr (LPG == 4) step(std::integral_constant<int, 1>{});
    uint32_t sbits = 0;
    int flags = 0;
    bool slow = false;
    if (maxmag >= 0x7F80u) {  // an Inf or NaN weight
      sbits = 0x7E00;
      flags = kDevNonfinite;
    } else {
      const float E = fmaf(acc, 0x1p-19f, 0x1p-118f);
      constexpr float kInvG = 1.0f / G;
      const uint32_t qlo = __half_as_ushort(__float2half_rn(fmaxf(acc - E, 0.f) * kInvG));
      const uint32_t qhi = __half_as_ushort(__float2half_rn((acc + E) * kInvG));
      if (qlo == qhi) {
        sbits = qlo;
        if (sbits >= 0x7C00u) {
          sbits = 0x7C00;
          flags = kDevScaleOverflow;
        }
      } else {
        slow = true;
      }
    }

    // Exact path, taken by the whole wave when one of its groups needs it
    // (its shuffles need every lane): a fixed-point sum anchored at the
    // group's largest exponent (that of its largest magnitude), and the
    // 320-bit sum when that window is not enough.
    if (__any(slow)) {
      const uint32_t sbits_fast = sbits;
      const int flags_fast = flags;
      const uint32_t Emax = maxmag >> 7;  // group maximum, after the butterfly
      const int emax = Emax ? (int)Emax - 1 : 0;
      const bool nonfinite = Emax == 0xFFu;

      // fixed-point sum anchored at emax
      uint64_t T = 0;
      uint32_t inexact = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t u = (i & 1) ? (m2[i >> 1] >> 16) : (m2[i >> 1] & 0xFFFFu);
        const uint32_t E = u >> 7;
        const uint64_t sig = E ? 128u + (u & 0x7Fu) : (u & 0x7Fu);
        const int e = E ? (int)E - 1 : 0;
        const int sh = e - emax + kWin;
        if (sh >= 0) {
          T += sig << sh;
        } else if (sh > -8) {
          T += sig >> (-sh);
          inexact |= (sig & ((1ull << (-sh)) - 1)) != 0;
        } else {
          inexact |= sig != 0;
        }
      }
#pragma unroll
      for (int m = 1; m < LPG; m <<= 1) {
        T += shfl_xor_u64(T, m);
        inexact |= shfl_xor_u32(inexact, m);
      }

      // one rounding of the mean to fp16; the true sum lies in [T, T + G) units
      // of 2^(emax - 181) and the mean in units of 2^-24 is that times
      // 2^(emax - 157 - log2 G)
      sbits = 0;
      flags = 0;
      bool need_exact = false;
      if (nonfinite) {
        sbits = 0x7E00;
        flags = kDevNonfinite;
      } else {
        const int sh = emax - 157 - LOG2G;
        bool ovf;
        sbits = f16_bits_of_fixed(T, sh, &ovf);
        if (inexact) {
          bool ovf2;
          const uint32_t hi = f16_bits_of_fixed(T + (uint64_t)G, sh, &ovf2);
          need_exact = hi != sbits;
        }
        if (ovf && !need_exact) flags = kDevScaleOverflow;
      }
      if (need_exact && active && sub == 0) {
        bool ovf;
        sbits = f16_scale_exact(w + gi * G, G, LOG2G, &ovf);
        flags = ovf ? kDevScaleOverflow : 0;
      }
      const int leader = qg * LPG;
      sbits = (uint32_t)__shfl((int)sbits, leader, kWave);
      flags = __shfl(flags, leader, kWave);
      if (!slow) {
        sbits = sbits_fast;
        flags = flags_fast;
      }
    }

    // Codes: |w| > s/2, decided on bit patterns.  For a bf16 magnitude m
    // (fp32 bits m << 16) and the fp32 bits H of s/2, (m << 16) > H exactly
    // when m > H >> 16, so two weights are compared at once as 16-bit halves
    // (a saturating subtraction is non-zero exactly when m > H >> 16).  The
    // digit is 1 + t - 2 t sign with t = [m > H >> 16]; flagged groups keep
    // every digit at 1 (code 0).
    const uint32_t half_bits =
        __float_as_uint(__half2float(__ushort_as_half((unsigned short)sbits)) * 0.5f);
    const u16x2 hb = as_u16x2((half_bits >> 16) * 0x00010001u);
    const u16x2 one = as_u16x2(0x00010001u);
    uint32_t d2[16];  // digits 2i, 2i+1 in the low bytes of the halves
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u16x2 t = __builtin_elementwise_min(
          __builtin_elementwise_sub_sat(as_u16x2(m2[i]), hb), one);
      const u16x2 sg = as_u16x2((raw[i] >> 15) & 0x00010001u);
      const u16x2 ts = t & sg;
      d2[i] = flags ? 0x00010001u : as_u32(one + t - (ts + ts));
    }
    uint32_t db[9];  // digits as bytes: db[j] holds digits 4j .. 4j+3
#pragma unroll
    for (int j = 0; j < 8; ++j) db[j] = __builtin_amdgcn_perm(d2[2 * j + 1], d2[2 * j], 0x06040200u);

    if constexpr (MODE == kPack2) {
      // four 2-bit fields d = c + 1 a byte, first weight lowest: this lane's
      // 32 weights are 8 bytes of the group's G/4, stored as four halves
      // (the buffer is 2-byte aligned)
      uint32_t by[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) by[j] = __builtin_amdgcn_udot4(db[j], 0x40100401u, 0u, false);
      if (active) {
        uint16_t *dst = reinterpret_cast<uint16_t *>(packed + gi * (G / 4) + sub * 8);
#pragma unroll
        for (int h = 0; h < 4; ++h) dst[h] = (uint16_t)(by[2 * h] | (by[2 * h + 1] << 8));
        if (sub == 0) {
          scales[gi] = (uint16_t)sbits;
          if (flags && d_status) atomicOr(d_status, flags);
        }
      }
      continue;
    }
    // Five digits a byte, base 3, first weight least significant.  Byte b of
    // the group holds digits 5b .. 5b+4 and is written by the lane with
    // 32 sub <= 5b < 32 sub + 32 (6 or 7 bytes a lane, every byte once).  Its
    // last byte reaches up to 4 digits into the next lane's, fetched by one
    // DPP shift within the group's lanes; past the group's last lane they are
    // padding digits 1 (code 0).  The lane's window is first shifted by p0
    // digits so that its own bytes start at window digit 0.
    const uint32_t next =
        (uint32_t)__builtin_amdgcn_update_dpp((int)0x01010101, (int)db[0], 0x101, 0xF, 0xF, false);
    db[8] = sub == LPG - 1 ? 0x01010101u : next;
    const int b0 = (kWPL * sub + 4) / 5;           // the lane's first byte
    const uint32_t p0 = (uint32_t)(5 * b0 - kWPL * sub);  // its first digit: 0..4
    const int nb = (kWPL * sub + kWPL - 1) / 5 - b0 + 1;  // its bytes: 6 or 7
    // (alignbyte shifts by 0..3 bytes; a shift of 4 is the next dword)
    uint32_t wd[9];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wd[j] = p0 == 4u ? db[j + 1] : __builtin_amdgcn_alignbyte(db[j + 1], db[j], p0);
    wd[8] = p0 == 4u ? 0x01010101u : __builtin_amdgcn_alignbyte(0x01010101u, db[8], p0);
    if (active) {
#pragma unroll
      for (int k = 0; k < 7; ++k) {
        const int q0 = 5 * k;  // window digit of the byte's first digit
        const uint32_t four = (q0 & 3) ? __builtin_amdgcn_alignbyte(wd[(q0 >> 2) + 1], wd[q0 >> 2],
                                                                    (uint32_t)(q0 & 3))
                                       : wd[q0 >> 2];
        const uint32_t fifth = (wd[(q0 + 4) >> 2] >> (8 * ((q0 + 4) & 3))) & 0xFFu;
        const uint32_t byte = __builtin_amdgcn_udot4(four, 0x1B090301u, 81u * fifth, false);
        if (k < nb) packed[gi * B + b0 + k] = (uint8_t)byte;
      }
      if (sub == 0) {
        scales[gi] = (uint16_t)sbits;
        if (flags && d_status) atomicOr(d_status, flags);
      }
    }
  }
}

// The QAT forward on 8 weights a lane (G/8 lanes a group, one 16-byte load
// and one 16-byte store each, so a wave's loads and stores are contiguous):
// the same scale computation as quantize_pack_kernel (an fp32 sum over an
// in-order chain of 8 and a butterfly over the group's lanes, the exact path
// when the interval test fails), then w_hat = bf16(c * s) written where the
// weights were read.  Its writes are as large as its reads, and 16-byte lanes
// 64 bytes apart (32 weights a lane) made it 12% slower.
template <int G>
__global__ __launch_bounds__(kBlock) void fake_quantize_kernel(const QuantBatch args,
                                                               int64_t total_groups,
                                                               int32_t *__restrict__ d_status) {
  const uint16_t *__restrict__ w = args.w[blockIdx.y];
  uint16_t *__restrict__ scales = args.scales[blockIdx.y];
  uint16_t *__restrict__ w_hat = args.w_hat[blockIdx.y];
  constexpr int LPG = G / 8;               // lanes per group
  constexpr int GPC = 512 / G;             // groups per chunk
  constexpr int LOG2G = (G == 64) ? 6 : 7;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane % LPG;
  const int qg = lane / LPG;
  const int64_t nchunks = (total_groups + GPC - 1) / GPC;

  for (int64_t base = (int64_t)blockIdx.x * kWavesPerBlock; base < nchunks;
       base += (int64_t)gridDim.x * kWavesPerBlock) {
    const int64_t chunk = base + wv;
    const int64_t gi = chunk * GPC + qg;
    const bool active = chunk < nchunks && gi < total_groups;

    uint32_t raw[4] = {0, 0, 0, 0};
    if (active) {
      const uint4 v = load_streamed(w + gi * G + sub * 8);
      raw[0] = v.x; raw[1] = v.y; raw[2] = v.z; raw[3] = v.w;
    }
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) { h[2 * i] = raw[i] & 0xFFFFu; h[2 * i + 1] = raw[i] >> 16; }

    // Fast path.  The sum of |w| in fp32: each lane adds its 8 magnitudes in
    // order, then an xor butterfly over the group's LPG lanes (fp32 addition
    // commutes, so every lane ends with the same sum S_hat).  Along any path
    // there are at most 7 + log2(LPG) <= 11 rounded additions of non-negative
    // terms, so |S_hat - S| <= 11 * 2^-24 * S, plus at most G * 2^-126 should
    // subnormals be flushed.  With E = 2^-19 S_hat + 2^-118 the exact sum lies
    // in [S_hat - E, S_hat + E] even after the rounding of those two
    // operations; when both ends, divided by G, round to the same fp16 value,
    // so does the exact mean (rounding is monotonic).  Otherwise the group
    // takes the exact path below.
    float acc = 0.f;
    uint32_t maxmag = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t mag = h[i] & 0x7FFFu;
      maxmag = mag > maxmag ? mag : maxmag;
      acc += __uint_as_float(mag << 16);
    }
    auto step = [&](auto k) {
      acc += __uint_as_float(dpp_partner<decltype(k)::value>(__float_as_uint(acc)));
      const uint32_t o = dpp_partner<decltype(k)::value>(maxmag);
      maxmag = o > maxmag ? o : maxmag;
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    if constexpr (LPG == 16) step(std::integral_constant<int, 3>{});
    uint32_t sbits = 0;
    int flags = 0;
    bool slow = false;
    if (maxmag >= 0x7F80u) {  // an Inf or NaN weight
      sbits = 0x7E00;
      flags = kDevNonfinite;
    } else {
      const float E = fmaf(acc, 0x1p-19f, 0x1p-118f);
      constexpr float kInvG = 1.0f / G;
      const uint32_t qlo = __half_as_ushort(__float2half_rn(fmaxf(acc - E, 0.f) * kInvG));
      const uint32_t qhi = __half_as_ushort(__float2half_rn((acc + E) * kInvG));
      if (qlo == qhi) {
        sbits = qlo;
        if (sbits >= 0x7C00u) {
          sbits = 0x7C00;
          flags = kDevScaleOverflow;
        }
      } else {
        slow = true;
      }
    }

    // Exact path, taken by the whole wave when one of its groups needs it
    // (its shuffles need every lane): exponent maximum, a fixed-point sum
    // anchored at it, and the 320-bit sum when that window is not enough.
    if (__any(slow)) {
      const uint32_t sbits_fast = sbits;
      const int flags_fast = flags;
      // exponent maximum and non-finite flag over the group
      int emax = 0;
      uint32_t nonfinite = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t E = (h[i] >> 7) & 0xFFu;
        nonfinite |= (E == 0xFFu);
        const int e = E ? (int)E - 1 : 0;
        emax = e > emax ? e : emax;
      }
#pragma unroll
      for (int m = 1; m < LPG; m <<= 1) {
        const int o = (int)shfl_xor_u32((uint32_t)emax, m);
        emax = o > emax ? o : emax;
        nonfinite |= shfl_xor_u32(nonfinite, m);
      }

      // fixed-point sum anchored at the group's largest exponent
      uint64_t T = 0;
      uint32_t inexact = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t u = h[i] & 0x7FFFu;
        const uint32_t E = u >> 7;
        const uint64_t sig = E ? 128u + (u & 0x7Fu) : (u & 0x7Fu);
        const int e = E ? (int)E - 1 : 0;
        const int sh = e - emax + kWin;
        if (sh >= 0) {
          T += sig << sh;
        } else if (sh > -8) {
          T += sig >> (-sh);
          inexact |= (sig & ((1ull << (-sh)) - 1)) != 0;
        } else {
          inexact |= sig != 0;
        }
      }
#pragma unroll
      for (int m = 1; m < LPG; m <<= 1) {
        T += shfl_xor_u64(T, m);
        inexact |= shfl_xor_u32(inexact, m);
      }

      // one rounding of the mean to fp16; the true sum lies in [T, T + G) units
      // of 2^(emax - 181) and the mean in units of 2^-24 is that times
      // 2^(emax - 157 - log2 G)
      sbits = 0;
      flags = 0;
      bool need_exact = false;
      if (nonfinite) {
        sbits = 0x7E00;
        flags = kDevNonfinite;
      } else {
        const int sh = emax - 157 - LOG2G;
        bool ovf;
        sbits = f16_bits_of_fixed(T, sh, &ovf);
        if (inexact) {
          bool ovf2;
          const uint32_t hi = f16_bits_of_fixed(T + (uint64_t)G, sh, &ovf2);
          need_exact = hi != sbits;
        }
        if (ovf && !need_exact) flags = kDevScaleOverflow;
      }
      if (need_exact && active && sub == 0) {
        bool ovf;
        sbits = f16_scale_exact(w + gi * G, G, LOG2G, &ovf);
        flags = ovf ? kDevScaleOverflow : 0;
      }
      const int leader = qg * LPG;
      sbits = (uint32_t)__shfl((int)sbits, leader, kWave);
      flags = __shfl(flags, leader, kWave);
      if (!slow) {
        sbits = sbits_fast;
        flags = flags_fast;
      }
    }

    // codes: |w| > s/2, compared as ordered fp32 bit patterns (exact, no
    // denormal flushing involved); flagged groups keep all codes at 0
    const uint32_t half_bits =
        __float_as_uint(__half2float(__ushort_as_half((unsigned short)sbits)) * 0.5f);
    uint64_t dig = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t mag = (h[i] & 0x7FFFu) << 16;
      uint32_t d = 1;
      if (!flags && mag > half_bits) d = (h[i] & 0x8000u) ? 0u : 2u;
      dig |= (uint64_t)d << (8 * i);
    }

    {
      // w_hat of the 8 weights: a pair takes bytes 2d, 2d+1 of {hi, lo}
      // per digit d (0..1 is -s, 2..3 +0, 4..5 +s); a flagged group is +0
      const uint32_t sb = flags ? 0u : bf16_of_f16(sbits);
      const uint32_t lo = flags ? 0u : (sb ^ 0x8000u);  // s >= 0: -s | +0
      const uint32_t hi = sb | (sb << 16);
      uint32_t out[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t pair = (uint32_t)((dig >> (16 * k)) & 0xFFu) |
                              ((uint32_t)((dig >> (16 * k + 8)) & 0xFFu) << 16);
        out[k] = __builtin_amdgcn_perm(hi, lo, pair * 0x0202u + 0x01000100u);
      }
      if (active) {
        store_streamed(w_hat + gi * G + sub * 8, out[0], out[1], out[2], out[3]);
        if (sub == 0) {
          if (scales) scales[gi] = (uint16_t)sbits;
          if (flags && d_status) atomicOr(d_status, flags);
        }
      }
    }

  }
}


// ---------------------------------------------------------------------------
// unpack: one thread per 16 consecutive codes of a group (G % 16 == 0), one
// 16-byte store, so a wave writes 1 KB contiguously.  The 16 codes lie in
// four bytes of the group, read from the one or two aligned dwords holding
// them (both hold bytes of the group, so no read leaves the buffer's
// pages).  A 256-entry LDS table gives each byte's digits as 2-bit fields;
// each 4 digits are spread into the 4 selector bytes of one v_perm_b32 that
// picks 0xFF, 0x00 or 0x01 (codes -1, 0, 1).  U items per thread and pass,
// their loads issued before any is decoded.
// ---------------------------------------------------------------------------
struct UnpackBatch {
  const uint8_t *packed[kQuantMaxBatch];
  int8_t *codes[kQuantMaxBatch];
};

template <int G, int U>
__global__ __launch_bounds__(kBlock) void unpack_kernel(const UnpackBatch args, uint64_t total,
                                                        int32_t *__restrict__ d_status) {
  const uint8_t *__restrict__ packed = args.packed[blockIdx.y];
  int8_t *__restrict__ codes = args.codes[blockIdx.y];
  constexpr int TPG = G / 16;                 // threads per group
  constexpr int B = bytes_per_group(G);
  constexpr int NPAD = 5 * B - G;             // padding trits, in the group's last byte
  constexpr uint32_t kPadMask = (1u << (2 * NPAD)) - 1u;
  constexpr uint32_t kPadZero = 0x5555u & kPadMask;

  __shared__ uint32_t lut[256];
  lut[threadIdx.x] = digit_entry(threadIdx.x);
  __syncthreads();

  const uint32_t pmis = (uint32_t)(reinterpret_cast<uintptr_t>(packed) & 3u);
  const uint32_t *__restrict__ pw = reinterpret_cast<const uint32_t *>(packed - pmis);
  const bool a16 = (reinterpret_cast<uintptr_t>(codes) & 15u) == 0;
  int flags = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t t0 = (uint64_t)blockIdx.x * kBlock + threadIdx.x; t0 < total; t0 += U * stride) {
    uint32_t w0[U], w1[U], sh[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint64_t t = t0 + u * stride;
      t = t < total ? t : total - 1;          // past the end: reload the last item, store nothing
      const uint64_t gi = t / TPG;
      const int p0 = (int)(t % TPG) * 16;
      const uint64_t r = gi * B + p0 / 5 + pmis;
      w0[u] = pw[r >> 2];
      w1[u] = pw[(r + 3) >> 2];
      sh[u] = 8u * (uint32_t)(r & 3u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t t = t0 + u * stride;
      if (t >= total) break;
      const uint64_t gi = t / TPG;
      const int p0 = (int)(t % TPG) * 16;
      const int o = p0 - 5 * (p0 / 5);
      const uint32_t bytes = (uint32_t)((((uint64_t)w1[u] << 32) | w0[u]) >> sh[u]);
      const uint32_t e0 = lut[bytes & 0xFFu], e1 = lut[(bytes >> 8) & 0xFFu];
      const uint32_t e2 = lut[(bytes >> 16) & 0xFFu], e3 = lut[bytes >> 24];
      if ((e0 | e1 | e2 | e3) & kLutInvalid) flags |= kDevInvalidByte;
      const uint64_t D = (uint64_t)((e0 & 0x3FFu) | ((e1 & 0x3FFu) << 10) | ((e2 & 0x3FFu) << 20)) |
                         ((uint64_t)(e3 & 0x3FFu) << 30);
      const uint64_t d = D >> (2 * o);        // digits of codes p0 .., then the next ones
      if (p0 + 16 == G && (((uint32_t)(d >> 32)) & kPadMask) != kPadZero)
        flags |= kDevBadPadding;
      uint32_t out[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t x = ((uint32_t)d >> (8 * k)) & 0xFFu;       // 4 digits
        uint32_t y = (x | (x << 12)) & 0x000F000Fu;                 // d0 d1 | d2 d3
        y = (y | (y << 6)) & 0x03030303u;                          // one digit per byte
        out[k] = __builtin_amdgcn_perm(0u, 0x000100FFu, y);         // -1, 0, +1
      }
      int8_t *dst = codes + gi * G + p0;
      if (a16) {
        store_streamed(dst, out[0], out[1], out[2], out[3]);
      } else {  // codes only 8-byte aligned (the ABI's minimum)
        reinterpret_cast<uint2 *>(dst)[0] = make_uint2(out[0], out[1]);
        reinterpret_cast<uint2 *>(dst)[1] = make_uint2(out[2], out[3]);
      }
    }
  }
  if (flags && d_status) atomicOr(d_status, flags);
}

int grid_for(int64_t work_items, int64_t per_block, int64_t cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

// count problems of one shape, up to kQuantMaxBatch per launch; each
// problem gets the same number of blocks (at most kMaxBlocks in a launch).
void launch_quant_batched(int count, const uint16_t *const *ws, int64_t N, int64_t K, int G,
                          uint8_t *const *packeds, uint16_t *const *scales,
                          uint16_t *const *w_hats, int32_t *d_status, hipStream_t stream,
                          bool two_bit) {
  const int64_t total_groups = N * (K / G);
  const bool fake = w_hats != nullptr;
  // chunks of 2048 weights a wave (packing) or 512 (the QAT forward)
  const int64_t per = fake ? 512 : kChunk;
  const int64_t nchunks = (total_groups * G + per - 1) / per;
  for (int c0 = 0; c0 < count; c0 += kQuantMaxBatch) {
    const int n = count - c0 < kQuantMaxBatch ? count - c0 : kQuantMaxBatch;
    QuantBatch a{};
    for (int i = 0; i < n; ++i) {
      a.w[i] = ws[c0 + i];
      a.packed[i] = packeds ? packeds[c0 + i] : nullptr;
      a.scales[i] = scales ? scales[c0 + i] : nullptr;
      a.w_hat[i] = fake ? w_hats[c0 + i] : nullptr;
    }
    const dim3 grid(grid_for(nchunks, kWavesPerBlock, kMaxBlocks / n), n);
    if (G == 64) {
      if (fake)
        hipLaunchKernelGGL((fake_quantize_kernel<64>), grid, dim3(kBlock), 0, stream, a,
                           total_groups, d_status);
      else if (two_bit)
        hipLaunchKernelGGL((quantize_pack_kernel<64, kPack2>), grid, dim3(kBlock), 0, stream, a,
                           total_groups, d_status);
      else
        hipLaunchKernelGGL((quantize_pack_kernel<64, kPack3>), grid, dim3(kBlock), 0, stream, a,
                           total_groups, d_status);
    } else {
      if (fake)
        hipLaunchKernelGGL((fake_quantize_kernel<128>), grid, dim3(kBlock), 0, stream, a,
                           total_groups, d_status);
      else if (two_bit)
        hipLaunchKernelGGL((quantize_pack_kernel<128, kPack2>), grid, dim3(kBlock), 0, stream,
                           a, total_groups, d_status);
      else
        hipLaunchKernelGGL((quantize_pack_kernel<128, kPack3>), grid, dim3(kBlock), 0, stream,
                           a, total_groups, d_status);
    }
  }
}

void launch_quantize_pack(const uint16_t *w, int64_t N, int64_t K, int G, uint8_t *packed,
                          uint16_t *scales, int32_t *d_status, hipStream_t stream) {
  launch_quant_batched(1, &w, N, K, G, &packed, &scales, nullptr, d_status, stream, false);
}

void launch_fake_quantize(const uint16_t *w, int64_t N, int64_t K, int G, uint16_t *w_hat,
                          uint16_t *scales, int32_t *d_status, hipStream_t stream) {
  launch_quant_batched(1, &w, N, K, G, nullptr, &scales, &w_hat, d_status, stream, false);
}

template <int G, int U>
void launch_unpack_u(const UnpackBatch &a, int n, uint64_t total, int32_t *d_status,
                     hipStream_t stream) {
  uint64_t blocks = (total + kBlock * U - 1) / (kBlock * U);
  const uint64_t cap = (uint64_t)(kMaxBlocks / n);
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((unpack_kernel<G, U>), dim3((unsigned)blocks, (unsigned)n), dim3(kBlock), 0,
                     stream, a, total, d_status);
}

template <int G>
void launch_unpack_g(const UnpackBatch &a, int n, uint64_t total, int32_t *d_status,
                     hipStream_t stream) {
  // the most items per thread that still leaves 2048 blocks (8 per CU)
  const uint64_t b4 = (total + kBlock * 4 - 1) / (kBlock * 4) * (uint64_t)n;
  if (b4 >= 2048)
    launch_unpack_u<G, 4>(a, n, total, d_status, stream);
  else if (2 * b4 >= 2048)
    launch_unpack_u<G, 2>(a, n, total, d_status, stream);
  else
    launch_unpack_u<G, 1>(a, n, total, d_status, stream);
}

void launch_unpack_batched(int count, const uint8_t *const *packeds, int64_t N, int64_t K, int G,
                           int8_t *const *codes, int32_t *d_status, hipStream_t stream) {
  const uint64_t total = (uint64_t)N * (uint64_t)K / 16;  // items of 16 codes per problem
  for (int c0 = 0; c0 < count; c0 += kQuantMaxBatch) {
    const int n = count - c0 < kQuantMaxBatch ? count - c0 : kQuantMaxBatch;
    UnpackBatch a{};
    for (int i = 0; i < n; ++i) {
      a.packed[i] = packeds[c0 + i];
      a.codes[i] = codes[c0 + i];
    }
    if (G == 64)
      launch_unpack_g<64>(a, n, total, d_status, stream);
    else
      launch_unpack_g<128>(a, n, total, d_status, stream);
  }
}

void launch_unpack(const uint8_t *packed, int64_t N, int64_t K, int G, int8_t *codes,
                   int32_t *d_status, hipStream_t stream) {
  launch_unpack_batched(1, &packed, N, K, G, &codes, d_status, stream);
}

}  // namespace tq
