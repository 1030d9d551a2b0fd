/*
 * tq_probe.h -- measurement probes in libtq.so: the rates this GPU reaches
 * on plain work, against which the hot path's kernels are reported beside
 * the published peaks (tiny-llm "Week 2 Day 3: Quantize the Model",
 * "Revisit the Decode Roofline": decode is bounded by the bytes streamed
 * per second, prefill by the matrix units).  They compute nothing of the
 * method.
 *
 * Ownership and streams as in tq.h: device pointers owned by the caller,
 * every call only enqueues work on `stream`.  Return TQ_OK (0), or a
 * negative tq_status with nothing enqueued.
 */
#ifndef TQ_PROBE_H
#define TQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of `buf` once, as 16-byte loads (a lane's loads 16
 * bytes apart across a wave, eight in flight per lane), with `grid` blocks of
 * 512 threads striding over the buffer.  Nothing is written unless the
 * XOR of everything read equals a value no test data holds; `sink` (one
 * uint32 per thread of the grid, grid * 512 entries) receives it then.
 *   buf    16-byte aligned; bytes a positive multiple of 16, below 2^40
 *   grid   1 .. 65535
 * TQ_ERR_NULL, TQ_ERR_ALIGN or TQ_ERR_SHAPE otherwise.
 */
int tq_probe_read_stream(const void *buf, int64_t bytes, int grid, uint32_t *sink, void *stream);

/*
 * Every wave of `grid` blocks of 512 threads runs `iters` rounds of eight
 * independent v_mfma_f32_16x16x32_bf16 on register operands (16384 flops
 * each), so the work is grid * 8 * iters * 8 * 16384 flops.  The eight fp32
 * results of lane 0 of each wave are written to `sink` (grid * 8 * 8
 * floats) only if they sum to a value the inputs cannot give.
 *   iters  1 .. 2^24;  grid 1 .. 65535
 * TQ_ERR_NULL or TQ_ERR_SHAPE otherwise.
 */
int tq_probe_mfma_bf16(int64_t iters, int grid, float *sink, void *stream);

/*
 * LDS table reads in the layout of the decode kernels' code tables: each of
 * `grid` blocks of 512 threads fills a 64 KB table (entry e of copy j at
 * byte e * 256 + j * 16), then every thread performs `iters` iterations of
 * eight 16-byte reads (ds_read_b128) from copy (thread % 16), at eight
 * entries drawn once per thread: grid * 512 * iters * 128 bytes read.
 * `sink` (grid * 512 uint32) is written only if the XOR of what was read
 * equals a value the table cannot give.  If `clocks` (two uint64, may be
 * NULL) is given, block 0's first thread stores the core-clock cycles and the
 * 10 ns ticks its loop took, so the caller can turn the rate into bytes per
 * cycle per CU.
 *   iters  1 .. 2^24;  grid 1 .. 65535
 * TQ_ERR_NULL or TQ_ERR_SHAPE otherwise.
 */
int tq_probe_lds_table(int iters, int grid, uint32_t *sink, unsigned long long *clocks,
                       void *stream);

/*
 * VALU issue rate: every wave of `grid` blocks of 512 threads runs `iters`
 * iterations of 16 steps of eight independent chains of one instruction,
 * kind 0 v_dot2_f32_bf16 or kind 1 v_perm_b32 (the decode GEMV's per-byte
 * instructions): grid * 8 * iters * 128 wave instructions.  `sink` and
 * `clocks` as for tq_probe_lds_table.
 *   kind 0 or 1;  iters 1 .. 2^24;  grid 1 .. 65535
 * TQ_ERR_NULL or TQ_ERR_SHAPE otherwise.
 */
int tq_probe_valu(int kind, int iters, int grid, uint32_t *sink, unsigned long long *clocks,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H */
