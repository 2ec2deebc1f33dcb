/*
 * moe_probe.h -- measurement probes of libmoe: the peaks that the layer's
 * kernels are compared against, measured on the device at hand rather than
 * taken from a data sheet.  Not part of the layer's computation.
 *
 * Conventions as in moe.h: device pointers, `stream` a hipStream_t passed as
 * void*, validation on the host, asynchronous enqueue, MOE_OK or a negative
 * MOE_E* code (text in moe_last_error()).  Nothing is allocated.
 */
#ifndef LIBMOE_MOE_PROBE_H
#define LIBMOE_MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a
 * multiple of 16) with 16-byte loads spread over every compute unit; each
 * workgroup folds what it read into one word of `sink` (uint32
 * [moe_probe_read_blocks(bytes)]), so that no load can be elided.  Timing
 * one launch (over a buffer larger than the last-level cache) gives the
 * achievable HBM read bandwidth. */
int moe_probe_read_blocks(size_t bytes);
int moe_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Dense matrix-core throughput: `blocks` workgroups of 4 waves, each wave
 * issuing `iters` rounds of 8 independent matrix instructions on register
 * operands, and storing its accumulators to `sink` (fp32 [blocks * 256 *
 * 32]).  kind: MOE_PROBE_BF16 (v_mfma_f32_16x16x32_bf16, the operand type of
 * the 2-bit formats' GEMMs), MOE_PROBE_F16 (v_mfma_f32_16x16x32_f16),
 * MOE_PROBE_F8F4 (v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 x E2M1
 * operands, the A8 path's instruction), and the 32 x 32 x 16 shapes of bf16
 * and f16 (4 instructions a round).  *flops_out gets the dense flops the
 * launch performs (2 M N K per instruction). */
enum {
  MOE_PROBE_BF16 = 0,
  MOE_PROBE_F16 = 1,
  MOE_PROBE_F8F4 = 2,
  MOE_PROBE_BF16_32 = 3, /* v_mfma_f32_32x32x16_bf16: 4 instructions per round */
  MOE_PROBE_F16_32 = 4   /* v_mfma_f32_32x32x16_f16 */
};
int moe_probe_mfma(int kind, int blocks, int iters, float *sink, double *flops_out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_MOE_PROBE_H */
