/*
 * maxsim_probe.h -- a measurement aid shipped beside libmaxsim.so, in its own
 * library (libmaxsim_probe.so); it also measures the vector-ALU issue rate.  It is not part of the MaxSim operation: it
 * measures the matrix-core rate this GPU sustains for the instructions the
 * MaxSim kernels use (v_mfma_f32_32x32x16_{f16,bf16}, v_mfma_i32_16x16x64_i8),
 * on operand data the caller supplies.  The data matters: with random
 * operands the board's power limit lowers the clock, so the sustained rate is
 * well below the published peak, which assumes the full clock.
 *
 * All pointers are device pointers owned by the caller; calls are
 * asynchronous on `stream` (a hipStream_t, NULL = default stream); the caller
 * times them (for example with events around the launch).
 */
#ifndef MAXSIM_PROBE_H
#define MAXSIM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MAXSIM_PROBE_F16 = 0, MAXSIM_PROBE_BF16 = 1, MAXSIM_PROBE_I8 = 2 };

/* Bytes of operand data one launch with `blocks` workgroups reads: per wave,
 * 12 x 64 lanes x 16 bytes (8 A fragments, 4 B fragments).  0 if blocks < 1. */
size_t maxsim_probe_operand_bytes(int32_t blocks);

/* Multiply-add operations x 2 one launch performs. */
double maxsim_probe_ops_per_launch(int32_t kind, int32_t blocks, int32_t iters);

/* Launch `blocks` workgroups of 8 waves; each wave runs 4 independent MFMA
 * accumulation chains for iters x 8 k-steps on its fragments of `operands`
 * (maxsim_probe_operand_bytes(blocks) bytes, 16-byte aligned) and writes one
 * float per thread to `sink` (blocks x 512 floats).
 * Returns 0, or 1 (NULL pointer), 2 (blocks or iters < 1), 3 (unknown kind),
 * 6 (launch failed). */
int maxsim_probe_mfma(int32_t kind, const void* operands, int32_t blocks, int32_t iters, float* sink, void* stream);

/* Vector-ALU lane-instructions one maxsim_probe_valu launch issues. */
double maxsim_probe_valu_lane_ops_per_launch(int32_t blocks, int32_t iters);

/* Launch `blocks` workgroups of 512 threads; each thread runs 8 independent
 * chains of fp32 fused multiply-adds (v_fmac_f32, one lane-instruction each)
 * for iters x 8 steps, on values read from `operands` (1024 floats), and
 * writes one float per thread to `sink` (blocks x 512 floats): the rate the
 * vector ALU issues plain (not packed) fp32 instructions.
 * Returns 0, or 1 (NULL pointer), 2 (blocks or iters < 1), 6 (launch failed). */
int maxsim_probe_valu(const float* operands, int32_t blocks, int32_t iters, float* sink, void* stream);

/* Plain streaming read of `bytes` (a multiple of 16, >= 16) of device memory
 * at `buf` by `blocks` workgroups of 256 threads, 16 bytes per load, grid-
 * stride; every thread writes one word to `sink` (blocks x 256 words): the
 * HBM read rate a simple kernel of the same size reaches.
 * Returns 0, or 1 (NULL pointer), 2 (bad blocks or bytes), 6 (launch failed). */
int maxsim_probe_read(const void* buf, size_t bytes, int32_t blocks, unsigned* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAXSIM_PROBE_H */
