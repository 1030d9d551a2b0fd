// tq_internal.h -- launchers shared between the C-ABI file and the kernel
// files of libtq.so.  Host code only sees these declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// Device status bits (numeric values fixed by include/tq.h).
constexpr int kDevNonfinite = 1;
constexpr int kDevScaleOverflow = 2;
constexpr int kDevInvalidByte = 4;
constexpr int kDevBadPadding = 8;

constexpr int bytes_per_group(int G) { return (G + 4) / 5; }

void launch_quantize_pack(const uint16_t *w, int64_t N, int64_t K, int G,
                          uint8_t *packed, uint16_t *scales, int32_t *d_status,
                          hipStream_t stream);

// Problems per batched quantize / QAT-forward / unpack launch.
constexpr int kQuantMaxBatch = 64;

// count same-shaped problems: quantize + pack (w_hats == nullptr) or the QAT
// forward (w_hats given; packeds unused; scales may be nullptr, or hold
// nullptr entries, to skip them).
// two_bit: pack 2-bit fields (four codes a byte, G/4 bytes a group) instead
// of base-3 bytes.
void launch_quant_batched(int count, const uint16_t *const *ws, int64_t N, int64_t K, int G,
                          uint8_t *const *packeds, uint16_t *const *scales,
                          uint16_t *const *w_hats, int32_t *d_status, hipStream_t stream,
                          bool two_bit);

// 2-bit format (tq_twobit.hip): codes, and the M = 1 decode GEMV of up to
// kQuantMaxBatch same-shaped problems a launch (K/64 <= 64).
void launch_unpack2(const uint8_t *packed, int64_t N, int64_t K, int G, int8_t *codes,
                    int32_t *d_status, hipStream_t stream);
bool gemv2_supported(int64_t N, int64_t K, int G);
// QAT forward from fp32 latent weights (tq_fake32.hip)
void launch_fake_quantize_f32_batched(int count, const float *const *ws, int64_t N, int64_t K,
                                      int G, float *const *w_hats, uint16_t *const *scales,
                                      int32_t *d_status, hipStream_t stream);
// 2-bit matmul on the matrix cores, any M and K (tq_twobit_mm.hip)
bool matmul2_supported(int64_t M, int64_t N, int64_t K, int G);
void launch_matmul2_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                            const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                            int64_t K, int G, int32_t *d_status, hipStream_t stream);
void launch_gemv2_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                          const uint16_t *const *scales, float *const *ys, int64_t N, int64_t K,
                          int G, int32_t *d_status, hipStream_t stream);
void launch_gemv2_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                          const uint16_t *const *scales, float *const *ys, const int64_t *Ns,
                          const int64_t *Ks, int G, int32_t *d_status, hipStream_t stream);

// W4A16 decode GEMV (tq_w4a16.hip)
bool w4a16_gemv_supported(int64_t N, int64_t K, int G);
void launch_w4a16_gemv_batched(int count, const uint16_t *const *xs,
                               const uint32_t *const *packeds, const uint16_t *const *scales,
                               const uint16_t *const *biases, uint16_t *const *ys, int64_t N,
                               int64_t K, int G, hipStream_t stream);
void launch_w4a16_gemv_grouped(int count, const uint16_t *const *xs,
                               const uint32_t *const *packeds, const uint16_t *const *scales,
                               const uint16_t *const *biases, uint16_t *const *ys,
                               const int64_t *Ns, const int64_t *Ks, int G, hipStream_t stream);

// W4A16 on the matrix cores, any M (tq_w4a16_gemm.hip): also the W4A16 GEMV's
// path for the shapes w4a16_gemv_supported() rejects.
bool w4a16_mfma_supported(int64_t M, int64_t N, int64_t K, int G);
void launch_w4a16_mfma(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                       const uint16_t *biases, int64_t M, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream);
void launch_w4a16_mfma_batched(int count, const uint16_t *const *xs,
                               const uint32_t *const *packeds, const uint16_t *const *scales,
                               const uint16_t *const *biases, int64_t M, int64_t N, int64_t K,
                               int G, uint16_t *const *ys, hipStream_t stream);

void launch_unpack_batched(int count, const uint8_t *const *packeds, int64_t N, int64_t K, int G,
                           int8_t *const *codes, int32_t *d_status, hipStream_t stream);

// QAT forward (tq_quant.hip): w_hat = bf16(c * s) straight from w; scales
// written only if not null.
void launch_fake_quantize(const uint16_t *w, int64_t N, int64_t K, int G, uint16_t *w_hat,
                          uint16_t *scales, int32_t *d_status, hipStream_t stream);

void launch_unpack(const uint8_t *packed, int64_t N, int64_t K, int G,
                   int8_t *codes, int32_t *d_status, hipStream_t stream);

// Decode to bf16 (tq_dequant.hip): w_hat[n,k] = bf16(c[n,k] * s[n,k/G]).
void launch_dequantize(const uint8_t *packed, const uint16_t *scales, int64_t N, int64_t K, int G,
                       uint16_t *w_hat, int32_t *d_status, hipStream_t stream);

// Problems per batched decode launch.
constexpr int kDequantMaxBatch = 64;

void launch_dequantize_batched(int count, const uint8_t *const *packeds,
                               const uint16_t *const *scales, uint16_t *const *w_hats, int64_t N,
                               int64_t K, int G, int32_t *d_status, hipStream_t stream);

void launch_gemv(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
                 int64_t M, int64_t N, int64_t K, int G, float *y,
                 int32_t *d_status, hipStream_t stream);

void launch_gemv_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                         const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                         int64_t K, int G, int32_t *d_status, hipStream_t stream);

// M = 1 decode kernel (tq_gemv_m1.hip), for the shapes it supports.
bool gemv_m1_supported(int64_t M, int64_t N, int64_t K);

void launch_gemv_m1(const uint16_t *x, const uint8_t *packed, const uint16_t *scales, int64_t N,
                    int64_t K, int G, float *y, int32_t *d_status, hipStream_t stream);

// Problems of any shapes the M = 1 kernel takes, grouped into launches by
// kernel configuration (problems in order within a group).
void launch_gemv_m1_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                            const uint16_t *const *scales, float *const *ys, const int64_t *Ns,
                            const int64_t *Ks, int G, int32_t *d_status, hipStream_t stream);

void launch_gemv_m1_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                            const uint16_t *const *scales, float *const *ys, int64_t N, int64_t K,
                            int G, int32_t *d_status, hipStream_t stream);

void launch_gemm(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
                 int64_t M, int64_t N, int64_t K, int G, float *y,
                 int32_t *d_status, hipStream_t stream);

// Problems per batched GEMM launch.
constexpr int kGemmMaxBatch = 64;

// G = 128, M >= 256: 256 x 128 tiles, 64-wide stages (tq_gemm_wide.hip),
// for launches of count same-shaped problems with enough tiles.
bool gemm_wide_supported(int count, int64_t M, int64_t N, int64_t K, int G);

void launch_gemm_wide(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                      const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                      int64_t K, int32_t *d_status, hipStream_t stream);

// The same kernel over the 2-bit format (four codes a byte, G/4 bytes a
// group): count same-shaped problems, under gemm_wide_supported's conditions.
void launch_gemm2_wide(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                       const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                       int64_t K, int32_t *d_status, hipStream_t stream);

// Problems of different N and K (shared M) in one persistent launch (per 128).
bool gemm_wide_grouped_supported(int count, int64_t M, const int64_t *Ns, const int64_t *Ks, int G);
void launch_gemm_wide_grouped(int count, const uint16_t *const *xs,
                              const uint8_t *const *packeds, const uint16_t *const *scales,
                              float *const *ys, int64_t M, const int64_t *Ns, const int64_t *Ks,
                              int32_t *d_status, hipStream_t stream);

void launch_gemm_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                         const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                         int64_t K, int G, int32_t *d_status, hipStream_t stream);

void launch_gemm_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                         const uint16_t *const *scales, float *const *ys, int64_t M,
                         const int64_t *Ns, const int64_t *Ks, int G, int32_t *d_status,
                         hipStream_t stream);

}  // namespace tq
