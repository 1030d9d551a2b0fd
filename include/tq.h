/*
 * tq.h -- C ABI of libtq.so: group-wise ternary weight quantization and the
 * packed-ternary x bf16-activation matmul, hand-written HIP for gfx950
 * (AMD Instinct MI355X).
 *
 * Format (precisit "pack-unpack-run" README, codec.py description, scale-rule
 * and payload-rate paragraphs):
 *   - W[N,K] is split along K into groups of G weights (K % G == 0).
 *   - Each group stores one fp16 scale s = mean |w| over the group, rounded
 *     once to fp16 (round half to even) from the exact sum.
 *   - Each weight stores a code c in {-1,0,1}: c = sign(w) if |w| > s/2,
 *     else 0 (|w| == s/2 is a tie and goes to 0).
 *   - Codes are packed five per byte as base-3 digits d = c + 1, the first
 *     weight of the five in the least significant digit:
 *       byte = sum_{i<5} (c[5b+i] + 1) * 3^i,
 *     each group separately byte-aligned in ceil(G/5) bytes, positions >= G
 *     padded with code 0.  Byte values 243..255 are invalid.
 *   - The reconstruction is w_hat = c * s; a zero scale makes a zero group.
 *   - Payload: 8 * (ceil(G/5) + 2) / G bits per weight (1.875 at G=64,
 *     1.750 at G=128).
 *
 * Layouts (all row-major, no padding between rows):
 *   w       uint16 [N][K]                 bf16 bit patterns
 *   packed  uint8  [N][K/G][ceil(G/5)]    group bytes, groups in K order
 *   scales  uint16 [N][K/G]               fp16 bit patterns
 *   codes   int8   [N][K]                 {-1, 0, 1}
 *   x       uint16 [M][K]                 bf16 bit patterns (finite)
 *   y       float  [M][N]                 fp32, y = x * W_hat^T
 *
 * Ownership: every pointer argument is a DEVICE pointer owned by the caller;
 * the library never allocates, frees or retains caller memory, and keeps no
 * per-call state.  Every call only enqueues work on `stream` (a hipStream_t,
 * or NULL for the null stream) and returns without synchronizing.  Calls are
 * thread-safe.
 *
 * Errors: argument errors detected on the host return a negative tq_status
 * and enqueue nothing.  Data errors found on the device are OR-ed into
 * *d_status (a device int32 the caller zeroes beforehand; d_status may be
 * NULL to skip reporting); read it after synchronizing the stream.  When a
 * bit is set, the outputs of the affected groups are as documented per call.
 *
 * Supported on the GPU: G in {64, 128}.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TQ_OK = 0,
    TQ_ERR_NULL = -1,    /* a required pointer is NULL                          */
    TQ_ERR_SHAPE = -2,   /* M, N or K < 1; K % G != 0; M > 16 in tq_gemv;       */
                         /* sizes whose byte counts overflow int64              */
    TQ_ERR_GROUP = -3,   /* G not in {64, 128}                                  */
    TQ_ERR_ALIGN = -4,   /* a pointer is not aligned as its call requires       */
    TQ_ERR_LAUNCH = -5   /* the HIP runtime reported an error at launch         */
} tq_status;

/* Device status bits. */
enum {
    TQ_DEV_NONFINITE = 1,      /* a weight (tq_quantize_pack) or a scale           */
                               /* (tq_dequantize) is Inf or NaN                    */
    TQ_DEV_SCALE_OVERFLOW = 2, /* a group mean rounds to >= 65520 (tq_quantize_pack)*/
    TQ_DEV_INVALID_BYTE = 4,   /* a packed byte is >= 243 (unpack, gemv, gemm)     */
    TQ_DEV_BAD_PADDING = 8     /* a padding trit is not code 0 (tq_unpack,         */
                               /* tq_dequantize)                                   */
};

/* Human-readable name of a tq_status value. */
const char *tq_status_string(int status);

/* Packed bytes of one row of K weights: (K/G) * ceil(G/5), each group
 * byte-aligned in ceil(G/5) bytes (precisit "pack-unpack-run" README,
 * codec.py description); 0 on bad arguments (K < 1, G < 1, K % G != 0).
 * Host-only helper, any G >= 1. */
int64_t tq_packed_row_bytes(int64_t K, int G);

/* Packed bytes of an [N,K] matrix: N * tq_packed_row_bytes(K, G); 0 on bad
 * arguments or when the count overflows int64 (host-only helper). */
int64_t tq_packed_bytes(int64_t N, int64_t K, int G);

/*
 * Quantize and pack W (steps: group scale, ternary codes, base-3 packing).
 * Source: precisit "pack-unpack-run" README, codec.py description and
 * scale-rule paragraph.
 *   w        [N,K] bf16, 16-byte aligned
 *   packed   [N, K/G, ceil(G/5)] bytes (any alignment)
 *   scales   [N, K/G] fp16 (2-byte aligned)
 * Group outputs under device errors: a group holding an Inf/NaN weight gets
 * scale 0x7E00 and all codes 0 (TQ_DEV_NONFINITE); a group whose mean rounds
 * to >= 65520 gets scale 0x7C00 and all codes 0 (TQ_DEV_SCALE_OVERFLOW).
 * Bit-exact and deterministic: results do not depend on launch shape.
 */
int tq_quantize_pack(const uint16_t *w, int64_t N, int64_t K, int G,
                     uint8_t *packed, uint16_t *scales,
                     int32_t *d_status, void *stream);

/*
 * Batched quantize + pack: `count` matrices of the same shape, each exactly
 * as tq_quantize_pack(ws[i], N, K, G, packeds[i], scales[i]), in one launch
 * per 64 matrices -- e.g. every weight of one shape in a checkpoint, which
 * one launch per matrix would leave to launch latency.
 *   ws, packeds, scales   HOST arrays of `count` DEVICE pointers, with the
 *                         layouts and alignments of tq_quantize_pack; read
 *                         during the call only
 *   count >= 0            (0 enqueues nothing)
 * Outputs must not overlap each other or any input.  Device status as
 * tq_quantize_pack; a NULL or misaligned pointer in any entry rejects the
 * whole call with nothing enqueued.
 */
int tq_quantize_pack_batched(int count, const uint16_t *const *ws, int64_t N, int64_t K, int G,
                             uint8_t *const *packeds, uint16_t *const *scales,
                             int32_t *d_status, void *stream);

/*
 * QAT forward ("fake quantization"): the ternarized weights in bf16,
 *   w_hat[n,k] = bf16_rne(c[n,k] * s[n, k/G])
 * with s and c exactly as tq_quantize_pack computes them, in one pass that
 * reads w and writes w_hat (no packed bytes).  Equal, bit for bit, to
 * tq_quantize_pack followed by tq_dequantize on unflagged groups.
 * Source: Avenue README (introduction and closing remarks: BitNet-style
 * quantization-aware training keeps latent weights and ternarizes them in
 * the forward pass; a kernel could remove the training overhead), with the
 * scale and code rule of the precisit "pack-unpack-run" README.  The
 * backward pass is straight-through (the gradient of w_hat is passed to w
 * unchanged) and needs no kernel.
 *   w        [N,K] bf16, 16-byte aligned
 *   w_hat    [N,K] bf16 bit patterns, 16-byte aligned, overwritten
 *   scales   [N, K/G] fp16, 2-byte aligned, or NULL (not written)
 * A group with an Inf/NaN weight (TQ_DEV_NONFINITE) or a mean that rounds
 * to >= 65520 (TQ_DEV_SCALE_OVERFLOW) gets w_hat = +0, and its scale as
 * tq_quantize_pack stores it.  Bit-exact and deterministic.
 */
int tq_fake_quantize(const uint16_t *w, int64_t N, int64_t K, int G, uint16_t *w_hat,
                     uint16_t *scales, int32_t *d_status, void *stream);

/*
 * Batched QAT forward: `count` matrices of the same shape, each exactly as
 * tq_fake_quantize(ws[i], N, K, G, w_hats[i], scales ? scales[i] : NULL),
 * in one launch per 64 matrices -- e.g. every projection of one shape in a
 * model, once per training step.
 *   ws, w_hats   HOST arrays of `count` DEVICE pointers (16-byte aligned)
 *   scales       NULL, or a HOST array of `count` DEVICE pointers (each
 *                2-byte aligned, or NULL to skip that matrix's scales)
 * Errors and device status as tq_fake_quantize; a NULL or misaligned
 * pointer in any entry rejects the whole call with nothing enqueued.
 */
int tq_fake_quantize_batched(int count, const uint16_t *const *ws, int64_t N, int64_t K, int G,
                             uint16_t *const *w_hats, uint16_t *const *scales,
                             int32_t *d_status, void *stream);

/*
 * QAT forward from fp32 latent weights (Avenue README, introduction: BitNet-
 * style training keeps full-precision latent weights and ternarizes them in
 * the forward pass; scale and code rule of the precisit "pack-unpack-run"
 * README applied to the fp32 values):
 *   w_hat[n,k] = c[n,k] * s[n,k/G]   in fp32, exact (s is an fp16 value)
 * s = RNE_fp16(exact mean of |w| over the group), c = sign(w) if |w| > s/2
 * else 0.  Code 0 gives +0; code -1 with s = +0 gives -0.
 *   w        [N,K] fp32, 16-byte aligned
 *   w_hat    [N,K] fp32, 16-byte aligned, overwritten (may not alias w)
 *   scales   [N, K/G] fp16, 2-byte aligned, or NULL (not written)
 * A group with an Inf/NaN weight (TQ_DEV_NONFINITE, scale 0x7E00) or a mean
 * that rounds to >= 65520 (TQ_DEV_SCALE_OVERFLOW, scale 0x7C00) gets
 * w_hat = +0.  Bit-exact and deterministic.
 */
int tq_fake_quantize_f32(const float *w, int64_t N, int64_t K, int G, float *w_hat,
                         uint16_t *scales, int32_t *d_status, void *stream);

/* Batched form: `count` same-shaped matrices, each as tq_fake_quantize_f32
 * on ws[i], w_hats[i], scales ? scales[i] : NULL (HOST arrays of DEVICE
 * pointers, read during the call only), one launch per 64.  Errors as
 * tq_fake_quantize_f32; a NULL or misaligned pointer in any entry rejects the
 * whole call with nothing enqueued. */
int tq_fake_quantize_f32_batched(int count, const float *const *ws, int64_t N, int64_t K, int G,
                                 float *const *w_hats, uint16_t *const *scales,
                                 int32_t *d_status, void *stream);

/*
 * Decode packed bytes to codes and validate them.
 * Source: precisit "pack-unpack-run" README, codec.py description
 * (decoding; values 243..255 invalid; zero-trit padding).
 *   packed   [N, K/G, ceil(G/5)] bytes (any alignment)
 *   codes    [N,K] int8 {-1,0,1}, 8-byte aligned
 * An invalid byte sets TQ_DEV_INVALID_BYTE and decodes to code 0 at its five
 * positions; a padding trit other than code 0 sets TQ_DEV_BAD_PADDING.
 */
int tq_unpack(const uint8_t *packed, int64_t N, int64_t K, int G,
              int8_t *codes, int32_t *d_status, void *stream);

/*
 * Batched unpack: `count` same-shaped matrices, each exactly as
 * tq_unpack(packeds[i], N, K, G, codes[i]), one launch per 64.
 *   packeds, codes   HOST arrays of `count` DEVICE pointers (codes 8-byte
 *                    aligned); read during the call only
 * Errors and device status as tq_unpack; a NULL or misaligned pointer in any
 * entry rejects the whole call with nothing enqueued.
 */
int tq_unpack_batched(int count, const uint8_t *const *packeds, int64_t N, int64_t K, int G,
                      int8_t *const *codes, int32_t *d_status, void *stream);

/*
 * Decode packed codes and group scales to a bf16 weight matrix:
 *   w_hat[n,k] = bf16_rne(c[n,k] * s[n, k/G])
 * Source: precisit "pack-unpack-run" README, codec.py description (decoding
 * gives back c * s) and screen.py description (the decoder hands the
 * selected weights back as bf16).  The product is exact; its one rounding,
 * to nearest with ties to even, is the fp16 -> bf16 rounding of s.  Zeros
 * carry the IEEE sign of c * s (code 0 takes the sign of s).
 *   packed   [N, K/G, ceil(G/5)] bytes (any alignment)
 *   scales   [N, K/G] fp16, 2-byte aligned
 *   w_hat    [N,K] bf16 bit patterns, 16-byte aligned, overwritten
 * An invalid byte sets TQ_DEV_INVALID_BYTE and its five weights decode as
 * code 0; a padding trit other than code 0 sets TQ_DEV_BAD_PADDING; an Inf
 * or NaN scale sets TQ_DEV_NONFINITE and its group decodes to +0.
 * Bit-exact and deterministic.
 */
int tq_dequantize(const uint8_t *packed, const uint16_t *scales, int64_t N, int64_t K,
                  int G, uint16_t *w_hat, int32_t *d_status, void *stream);

/*
 * Batched decode to bf16: `count` matrices of the same shape, each exactly
 * as tq_dequantize(packeds[i], scales[i], N, K, G, w_hats[i]), in one
 * launch per 64 matrices -- e.g. every tensor of one shape in a package,
 * which one launch per tensor would leave mostly to launch ramp-up.
 *   packeds, scales, w_hats   HOST arrays of `count` DEVICE pointers, with
 *                             the layouts and alignments of tq_dequantize;
 *                             read during the call only
 *   count >= 0                (0 enqueues nothing)
 * The outputs must not overlap each other or any input.  Errors and device
 * status as tq_dequantize; a NULL or misaligned pointer in any entry
 * rejects the whole call with nothing enqueued.
 */
int tq_dequantize_batched(int count, const uint8_t *const *packeds,
                          const uint16_t *const *scales, uint16_t *const *w_hats,
                          int64_t N, int64_t K, int G, int32_t *d_status, void *stream);

/*
 * Decode GEMV / skinny matmul, 1 <= M <= 16:
 *   y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
 * with fp32 group partials scaled by the fp16 group scale and accumulated in
 * fp32 (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical
 * Formulation" and "Revisit the Decode Roofline": one-token decode streams
 * every packed weight once).
 *   x        [M,K] bf16, 16-byte aligned
 *   packed   [N, K/G, ceil(G/5)] bytes, 16-byte aligned
 *   scales   [N, K/G] fp16, 2-byte aligned
 *   y        [M,N] fp32, 4-byte aligned, overwritten
 * K is at most 4194304 (2^22); larger K returns TQ_ERR_SHAPE.  Results are
 * deterministic (a fixed summation order for given shapes).  M = 1 runs a
 * table-decode kernel with dot2 accumulation; 2 <= M <= 16 (and M = 1 shapes
 * that kernel does not take) run on the matrix cores.
 * Invalid packed bytes set TQ_DEV_INVALID_BYTE; their contribution is then
 * unspecified.  Accuracy: |y - y_exact| <= 1e-3 * sum_k |x[m,k] w_hat[n,k]|.
 */
int tq_gemv(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
            int64_t M, int64_t N, int64_t K, int G,
            float *y, int32_t *d_status, void *stream);

/*
 * Batched decode GEMV: `count` independent problems of the same shape, each
 * exactly as tq_gemv(xs[i], packeds[i], scales[i], M, N, K, G, ys[i]), run in
 * as few launches as possible (one per 128 problems at M = 1, per 64 above)
 * so that a stack of small matrices -- e.g. the same projection of every layer of a decoder -- streams
 * its packed weights without a kernel launch per matrix.
 *   xs, packeds, scales, ys   HOST arrays of `count` DEVICE pointers, with
 *                             the layouts and alignments of tq_gemv; read
 *                             during the call only
 *   count >= 0                (0 enqueues nothing)
 * The outputs ys[i] must not overlap each other or any input.  Errors and
 * device status as tq_gemv; a NULL or misaligned pointer in any entry rejects
 * the whole call with nothing enqueued.
 */
int tq_gemv_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                    const uint16_t *const *scales, float *const *ys,
                    int64_t M, int64_t N, int64_t K, int G,
                    int32_t *d_status, void *stream);

/*
 * Grouped decode GEMV: `count` independent M = 1 problems of any shapes,
 * problem i being tq_gemv(xs[i], packeds[i], scales[i], 1, Ns[i], Ks[i], G,
 * ys[i]), in as few launches as possible: problems whose shapes run the same
 * kernel configuration share a launch (up to 128 per launch), which shares
 * the chip among them in proportion to their sizes -- e.g. every projection
 * of a stack of decoder layers, whatever its shape, in one pass.  Results
 * are bit-identical to the single-problem calls.
 *   xs, packeds, scales, ys   HOST arrays of `count` DEVICE pointers, with
 *                             the layouts and alignments of tq_gemv
 *   Ns, Ks                    HOST arrays of `count` shapes
 *                             (all HOST arrays are read during the call only)
 *   count >= 0                (0 enqueues nothing)
 * The outputs ys[i] must not overlap each other or any input.  Errors and
 * device status as tq_gemv; a NULL or misaligned pointer or a bad shape in
 * any entry rejects the whole call with nothing enqueued.
 */
int tq_gemv_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                    const uint16_t *const *scales, float *const *ys,
                    const int64_t *Ns, const int64_t *Ks, int G,
                    int32_t *d_status, void *stream);

/*
 * Prefill matmul for any M >= 1 (tuned for M >= 512): the same result as
 * tq_gemv, computed with bf16 MFMA on dequantized code tiles (codes are exact
 * in bf16), fp32 group partials scaled by the fp16 group scale in fp32.
 * Source: tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical
 * Formulation" and the decode-roofline remark that prefill reuses each
 * weight tile across many rows and needs a matrix schedule.
 *   x        [M,K] bf16, 16-byte aligned
 *   packed   [N, K/G, ceil(G/5)] bytes (any alignment)
 *   scales   [N, K/G] fp16, 2-byte aligned
 *   y        [M,N] fp32, 4-byte aligned, overwritten
 * K is at most 4194304 (2^22); larger K returns TQ_ERR_SHAPE.
 * Invalid packed bytes set TQ_DEV_INVALID_BYTE; their contribution is then
 * unspecified.  Accuracy as tq_gemv.
 */
int tq_gemm(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
            int64_t M, int64_t N, int64_t K, int G,
            float *y, int32_t *d_status, void *stream);

/*
 * Batched prefill matmul: `count` independent problems of the same shape,
 * each exactly as tq_gemm(xs[i], packeds[i], scales[i], M, N, K, G, ys[i]),
 * in as few launches as possible (one per 64 problems) so that the tiles of
 * all problems share the chip -- e.g. the same projection of every layer of
 * a decoder, or the gate and up projections that read the same activations.
 * Results are bit-identical to the single-problem calls.
 *   xs, packeds, scales, ys   HOST arrays of `count` DEVICE pointers, with
 *                             the layouts and alignments of tq_gemm; read
 *                             during the call only
 *   count >= 0                (0 enqueues nothing)
 * The outputs ys[i] must not overlap each other or any input.  Errors and
 * device status as tq_gemm; a NULL or misaligned pointer in any entry rejects
 * the whole call with nothing enqueued.
 */
int tq_gemm_batched(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                    const uint16_t *const *scales, float *const *ys,
                    int64_t M, int64_t N, int64_t K, int G,
                    int32_t *d_status, void *stream);

/*
 * Grouped prefill matmul: `count` independent problems that share M but may
 * differ in N and K, each as tq_gemm(xs[i], packeds[i], scales[i], M, Ns[i],
 * Ks[i], G, ys[i]) -- e.g. every projection of a decoder's FFN stack over one
 * prompt batch (gate/up [N=I, K=H] and down [N=H, K=I]).  Where the 256 x 128
 * tile kernel takes every shape (G = 128, M >= 256) all problems share one
 * persistent launch per 128 problems, longest K first, so that no shape's
 * tail leaves the chip idle between launches; otherwise the problems run as
 * one tq_gemm_batched call per distinct shape.  Same tiny-llm passages as
 * tq_gemm.
 *   xs, packeds, scales, ys   HOST arrays of `count` DEVICE pointers with the
 *                             layouts and alignments of tq_gemm (problem i
 *                             has shape Ns[i] x Ks[i]); read during the call
 *   Ns, Ks                    HOST arrays of `count` sizes
 *   count >= 0                (0 enqueues nothing)
 * Accuracy as tq_gemm; the outputs must not overlap each other or any input.
 * Errors and device status as tq_gemm; any invalid entry rejects the whole
 * call with nothing enqueued.
 */
int tq_gemm_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packeds,
                    const uint16_t *const *scales, float *const *ys, int64_t M,
                    const int64_t *Ns, const int64_t *Ks, int G,
                    int32_t *d_status, void *stream);

/*
 * The 2-bit ternary format: codes in two bits each, four a byte.
 * Source: Avenue README (size note: model sizes counted for 2-bit packing)
 * and "Autoregressive Language Model on the 6502 Processor" (ternary
 * parameters packed four a byte).  Layout taken here:
 *   packed2  uint8 [N][K/G][G/4]   field f = c + 1 in bits 2i..2i+1 of byte
 *                                   b for weight 4b + i (first weight lowest);
 *                                   f = 3 is invalid
 *   scales   [N, K/G] fp16, as for the base-3 format (same scale, same codes)
 * 8 * (G/4 + 2) / G bits per weight: 2.25 at G = 64, 2.125 at G = 128.
 */

/* Quantize and pack to the 2-bit format (scale and codes exactly as
 * tq_quantize_pack).  w [N,K] bf16 16-byte aligned; packed2 [N, K/4] bytes,
 * 2-byte aligned; scales [N, K/G] fp16, 2-byte aligned.  Device status and
 * flagged-group outputs as tq_quantize_pack (flagged groups: codes 0). */
int tq_quantize_pack2(const uint16_t *w, int64_t N, int64_t K, int G, uint8_t *packed2,
                      uint16_t *scales, int32_t *d_status, void *stream);

/* Batched form: `count` same-shaped matrices, each as tq_quantize_pack2 on
 * ws[i], packed2s[i], scales[i] (HOST arrays of DEVICE pointers, read during
 * the call only), one launch per 64.  Errors as tq_quantize_pack2; a NULL or
 * misaligned pointer in any entry rejects the whole call. */
int tq_quantize_pack2_batched(int count, const uint16_t *const *ws, int64_t N, int64_t K, int G,
                              uint8_t *const *packed2s, uint16_t *const *scales,
                              int32_t *d_status, void *stream);

/* 2-bit packed -> codes int8 [N,K] {-1,0,1}.  packed2 4-byte aligned, codes
 * 16-byte aligned.  A field of 3 sets TQ_DEV_INVALID_BYTE and reads as 0. */
int tq_unpack2(const uint8_t *packed2, int64_t N, int64_t K, int G, int8_t *codes,
               int32_t *d_status, void *stream);

/*
 * Decode GEMV over the 2-bit format, M = 1:
 *   y[n] = sum_g s[n,g] * sum_{j<G} x[gG+j] * c[n, gG+j]
 * (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation").
 *   x [1,K] bf16 16-byte aligned; packed2 [N, K/4] 16-byte aligned; scales
 *   [N, K/G] fp16 2-byte aligned; y [N] fp32 4-byte aligned, overwritten
 * K <= 4096 (K/64 <= 64) with N < 2^28 runs a table-decode kernel; longer
 * rows run tq_gemm2's matrix-core kernel at M = 1 (its limits apply, else
 * TQ_ERR_SHAPE).  A field of 3 sets TQ_DEV_INVALID_BYTE and counts as code
 * 0.  Deterministic; accuracy as tq_gemv.
 */
int tq_gemv2(const uint16_t *x, const uint8_t *packed2, const uint16_t *scales, int64_t N,
             int64_t K, int G, float *y, int32_t *d_status, void *stream);

/* Batched form: `count` same-shaped problems, each as tq_gemv2 on xs[i],
 * packed2s[i], scales[i], ys[i] (HOST arrays of DEVICE pointers, read during
 * the call only), one launch per 128.  Errors as tq_gemv2; a NULL or
 * misaligned pointer in any entry rejects the whole call. */
int tq_gemv2_batched(int count, const uint16_t *const *xs, const uint8_t *const *packed2s,
                     const uint16_t *const *scales, float *const *ys, int64_t N, int64_t K,
                     int G, int32_t *d_status, void *stream);

/* Grouped form: `count` problems of their own shapes Ns[i] x Ks[i] (HOST
 * arrays, as the pointer arrays), each as tq_gemv2, in one launch per 128
 * problems.  Every problem must meet tq_gemv2's limits; the first that does
 * not, or a NULL or misaligned pointer in any entry, rejects the whole call
 * with that error.  Each row's result is bit-identical to tq_gemv2's. */
int tq_gemv2_grouped(int count, const uint16_t *const *xs, const uint8_t *const *packed2s,
                     const uint16_t *const *scales, float *const *ys, const int64_t *Ns,
                     const int64_t *Ks, int G, int32_t *d_status, void *stream);

/*
 * Matmul over the 2-bit format for any number of activation rows and any row
 * length, on the matrix cores (bf16 MFMA on the exact codes; fp32 group
 * partials scaled by the fp16 scale):
 *   y[m,n] = sum_g s[n,g] * sum_{j<G} x[m, gG+j] * c[n, gG+j]
 * (tiny-llm "Week 2 Day 3: Quantize the Model", "Mathematical Formulation";
 * format as tq_gemv2).
 *   x [M,K] bf16 16-byte aligned; packed2 [N, K/4] 2-byte aligned (16-byte
 *   for M = 1 with K <= 4096, which runs tq_gemv2's kernel); scales [N, K/G]
 *   fp16 2-byte aligned; y [M,N] fp32 4-byte aligned, overwritten
 * G is 64 or 128 (TQ_ERR_GROUP otherwise); K % G == 0, M * K * 2, N * K / 4
 * and N * K/G * 2 below 2^31, M <= 4194240, else TQ_ERR_SHAPE.  A field of 3
 * sets TQ_DEV_INVALID_BYTE and counts as code 0.  Deterministic; accuracy as
 * tq_gemv.
 */
int tq_gemm2(const uint16_t *x, const uint8_t *packed2, const uint16_t *scales, int64_t M,
             int64_t N, int64_t K, int G, float *y, int32_t *d_status, void *stream);

/* Batched form: `count` same-shaped problems, each as tq_gemm2 on xs[i],
 * packed2s[i], scales[i], ys[i] (HOST arrays of DEVICE pointers, read during
 * the call only), one launch per 64 problems.  count == 0 does nothing;
 * count < 0 is TQ_ERR_SHAPE; a NULL or misaligned pointer in any entry
 * rejects the whole call with nothing enqueued. */
int tq_gemm2_batched(int count, const uint16_t *const *xs, const uint8_t *const *packed2s,
                     const uint16_t *const *scales, float *const *ys, int64_t M, int64_t N,
                     int64_t K, int G, int32_t *d_status, void *stream);

/*
 * W4A16: group-wise affine 4-bit weights, bf16 activations and output
 * (tiny-llm "Week 2 Day 3: Quantize the Model": "Group-Wise Affine
 * Quantization", "Reconstruct a Stored Group", "Packed Storage Layout",
 * "Mathematical Formulation", "Computation Flow").
 *   x       [1,K] bf16, 16-byte aligned
 *   packed  [N, K/8] uint32, 16-byte aligned: weight 8p + i of a row in bits
 *           4i..4i+3 of its word p; codes q in [0, 15]
 *   scales, biases  [N, K/G] bf16, 2-byte aligned; either sign of scale
 *   y       [1,N] bf16, 2-byte aligned, overwritten
 *   y[n] = bf16_RNE( sum_k x[k] * (q[n,k] * s[n,k/G] + b[n,k/G]) ), the sum
 *   taken in fp32 as s * sum(x q) + b * sum(x) per group.
 * G is 64 or 128 (TQ_ERR_GROUP otherwise).  K <= 4096 (K/64 <= 64) with
 * N < 2^28 runs a table-decode kernel; longer rows run tq_w4a16_gemm's
 * matrix-core kernel at M = 1 (its limits apply, else TQ_ERR_SHAPE).  No data
 * errors exist in this format: every
 * code is valid, and Inf/NaN parameters or activations propagate to y.
 * Deterministic.  Accuracy: |y - y_exact| <= 1e-3 * sum_k |x| (|q s| + |b|)
 * before the final bf16 rounding.
 */
int tq_w4a16_gemv(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                  const uint16_t *biases, int64_t N, int64_t K, int G, uint16_t *y,
                  void *stream);

/*
 * W4A16 matmul for any number of activation rows, in the format of
 * tq_w4a16_gemv (tiny-llm "Week 2 Day 3: Quantize the Model": "Group-Wise
 * Affine Quantization", "Packed Storage Layout", "Mathematical
 * Formulation", "Computation Flow", "GPU Dispatch"):
 *   y[m,n] = bf16_RNE( sum_k x[m,k] * (q[n,k] * s[n,k/G] + b[n,k/G]) ),
 *   the sum taken in fp32 as s * sum(x q) + b * sum(x) per group, on the
 *   matrix cores (bf16 MFMA on the exact bf16 values of the codes).
 *   x       [M,K] bf16, 16-byte aligned
 *   packed  [N, K/8] uint32, 4-byte aligned, as tq_w4a16_gemv
 *   scales, biases  [N, K/G] bf16, 2-byte aligned
 *   y       [M,N] bf16, 2-byte aligned, overwritten
 * G is 64 or 128 (TQ_ERR_GROUP otherwise); K % G == 0, M * K * 2 and
 * N * K / 2 below 2^31 and M <= 4194240, else TQ_ERR_SHAPE.  M = 1 with K <=
 * 4096 runs tq_w4a16_gemv's kernel.  No data errors; Inf/NaN parameters or
 * activations propagate.  Deterministic; accuracy as tq_w4a16_gemv.
 */
int tq_w4a16_gemm(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                  const uint16_t *biases, int64_t M, int64_t N, int64_t K, int G, uint16_t *y,
                  void *stream);

/* Batched form: `count` same-shaped problems, each as tq_w4a16_gemm on
 * xs[i], packeds[i], scales[i], biases[i], ys[i] (HOST arrays of DEVICE
 * pointers, read during the call only), one launch per 64 problems (the
 * problems share the launch's grid, so a stack of matrices fills the GPU
 * where one matrix would not).  M = 1 with K <= 4096 runs
 * tq_w4a16_gemv_batched's kernel (packed then 16-byte aligned).  count == 0
 * does nothing; count < 0 is TQ_ERR_SHAPE; a NULL or misaligned pointer in
 * any entry rejects the whole call with nothing enqueued. */
int tq_w4a16_gemm_batched(int count, const uint16_t *const *xs, const uint32_t *const *packeds,
                          const uint16_t *const *scales, const uint16_t *const *biases,
                          int64_t M, int64_t N, int64_t K, int G, uint16_t *const *ys,
                          void *stream);

/* Batched form: `count` same-shaped problems, each as tq_w4a16_gemv on
 * xs[i], packeds[i], scales[i], biases[i], ys[i] (HOST arrays of DEVICE
 * pointers, read during the call only), one launch per 128.  Errors as
 * tq_w4a16_gemv; a NULL or misaligned pointer in any entry rejects the
 * whole call. */
int tq_w4a16_gemv_batched(int count, const uint16_t *const *xs, const uint32_t *const *packeds,
                          const uint16_t *const *scales, const uint16_t *const *biases,
                          uint16_t *const *ys, int64_t N, int64_t K, int G, void *stream);

/* Grouped form: `count` problems of their own shapes Ns[i] x Ks[i] (HOST
 * arrays, as the pointer arrays), each as tq_w4a16_gemv, in one launch per
 * 128 problems.  Every problem must meet tq_w4a16_gemv's limits; the first
 * that does not, or a NULL or misaligned pointer in any entry, rejects the
 * whole call with that error.  Each row's result is bit-identical to
 * tq_w4a16_gemv's. */
int tq_w4a16_gemv_grouped(int count, const uint16_t *const *xs, const uint32_t *const *packeds,
                          const uint16_t *const *scales, const uint16_t *const *biases,
                          uint16_t *const *ys, const int64_t *Ns, const int64_t *Ks, int G,
                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
