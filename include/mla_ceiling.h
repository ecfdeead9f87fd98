/*
 * libmla_ceiling -- measured ceilings of the part, for reading libmla's
 * roofline fractions against what the hardware sustains: a plain HBM
 * streaming read and back-to-back bf16 MFMA loops.  Not part of the decode
 * path.  Pointers are device pointers; every call only enqueues one kernel on
 * `stream` (a hipStream_t, NULL = default) and returns; the caller owns every
 * buffer.  Returns 0, -1 for a bad argument (nothing launched) or -4 when the
 * launch fails.
 */
#ifndef MLA_CEILING_H
#define MLA_CEILING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Work-groups (256 threads) a launch with blocks_per_cu per CU uses on the
 * current device: the CU count times blocks_per_cu (1..64); < 0 on error.
 * `sink` arguments below hold 256 entries per work-group. */
int mla_ceiling_blocks(int blocks_per_cu);

/* Reads `bytes` (a multiple of 16, 16-byte aligned) of `buf` once, with
 * 16-byte loads at a grid-wide stride, four in flight per thread; writes one
 * word per thread of sink (uint32). */
int mla_ceiling_stream_read(const void *buf, size_t bytes, int blocks_per_cu, unsigned *sink,
                            void *stream);

/* Every wave runs `iters` rounds of four independent bf16 MFMA chains:
 * shape 0 = v_mfma_f32_16x16x32_bf16, 1 = v_mfma_f32_32x32x16_bf16.  Writes
 * one float per thread of sink. */
int mla_ceiling_mfma(int shape, int iters, int blocks_per_cu, float *sink, void *stream);

/* Floating-point operations one mla_ceiling_mfma launch performs; < 0 on
 * error. */
double mla_ceiling_mfma_flops(int shape, int iters, int blocks_per_cu);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CEILING_H */
