/*
 * w4a8_probe.h -- roofline probes for MI355X (gfx950), used by the benchmark
 * to state what the hardware sustains next to its published peaks.  Not part
 * of the GEMM path.
 *
 * Conventions as in w4a8.h: device pointers, `stream` a hipStream_t as void*
 * (NULL = legacy default stream), asynchronous, W4A8_* status codes.  The
 * caller times the launches (hipEvents on `stream`).
 */
#ifndef W4A8_PROBE_H
#define W4A8_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * w4a8_probe_mfma -- a dense stream of v_mfma_scale_f32_16x16x128_f8f6f4 with
 * operand formats fmt_a, fmt_b (0 = FP8 E4M3, 4 = FP4 E2M1; the pairs
 * (4,0), (0,0), (4,4) are supported), eight independent accumulators per
 * wave, `blocks` workgroups of 256 threads, `iters` iterations per wave.
 * Each wave does iters * 8 MFMAs of 2*16*16*128 flops.  sink_dev: float
 * [blocks * 256], written (keeps the work live).  W4A8_ERR_SHAPE for an
 * unsupported pair or non-positive sizes.
 */
int w4a8_probe_mfma(int fmt_a, int fmt_b, int iters, int blocks, float* sink_dev, void* stream);

/*
 * w4a8_probe_mfma_data -- as w4a8_probe_mfma, but each thread's operands are
 * read from ops_dev: int32 [blocks * 256][16] (words 0-7 the A operand, 8-15
 * the B operand; for an FP4 operand only its first four words are used).
 * Filled with random bits it measures the sustained rate on realistic data,
 * which is well below the rate on constant operands.  Any bit pattern is
 * allowed (NaN codes only make NaN results).
 */
int w4a8_probe_mfma_data(int fmt_a, int fmt_b, int iters, int blocks, const int32_t* ops_dev,
                         float* sink_dev, void* stream);

/*
 * w4a8_probe_mfma_promote -- the grouped GEMM's MFMA-phase instruction
 * pattern without memory traffic: v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 A,
 * FP8 B) with a zero accumulator input, eight per iteration, each followed
 * (promote != 0) by the four fp32 FMAs that scale the partial of the MFMA
 * two back into an accumulator; promote == 0 issues the MFMAs alone.
 * `blocks` workgroups of 512 threads (two waves per SIMD), `iters`
 * iterations per wave, 8 MFMAs of 2*16*16*128 flops each.  ops_dev: int32
 * [blocks * 512][16] operand words (random bits for a realistic rate);
 * sink_dev: float [blocks * 512], written.
 */
int w4a8_probe_mfma_promote(int promote, int iters, int blocks, const int32_t* ops_dev, float* sink_dev,
                            void* stream);

/*
 * w4a8_probe_read -- reads `bytes` bytes from buf_dev once (16-byte loads,
 * grid-stride, eight loads in flight per lane) and writes one int to
 * sink_dev.  bytes must be a positive multiple of 16; buf_dev 16-byte aligned.
 */
int w4a8_probe_read(const void* buf_dev, size_t bytes, int blocks, int32_t* sink_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_PROBE_H */
