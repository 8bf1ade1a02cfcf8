/*
 * cca_probe.h - measurement probe shipped beside libcca (libcca_probe.so).
 *
 * Not part of the CCA hot path: a kernel that does nothing but dense bf16
 * matrix-core work, so that a benchmark can time, on the same chip, clocks and
 * power limit, the rate the matrix cores sustain on their own next to the
 * nominal peak.  The rate depends on the operand data (the chip's power, and so
 * its clock, follows the bits that toggle in the multipliers), so the operands
 * are drawn at random and rotate over several register sets, like the
 * streaming operands of a real kernel.
 */
#pragma once

#ifdef __cplusplus
extern "C" {
#endif

/*
 * cca_probe_mfma - enqueues one launch of the matrix-core probe on `stream`
 * (a hipStream_t; NULL is the default stream).  `blocks` workgroups of 8
 * waves (512 threads), two waves per SIMD; every wave runs `iters` rounds of
 * 16 v_mfma_f32_32x32x16_bf16 on two independent accumulator chains, with A/B
 * operands taken in turn from `operand_sets` register sets (1..4) of random
 * bf16 values in [-2, 2) (seeded by `seed`).  The launch executes
 * blocks * 8 * iters * 16 * 32768 floating-point operations.
 *   out: device buffer of blocks * 512 floats (the accumulators' sums, so that
 *        no work is dead); caller-owned.
 * Returns 0, 1 for an invalid argument (blocks < 1, iters < 1, operand_sets
 * outside 1..4, out NULL), or 1000 + the hipError_t when the launch fails.
 * Allocates nothing and does not synchronise.
 */
int cca_probe_mfma(float* out, int blocks, int iters, int operand_sets, unsigned seed, void* stream);

#ifdef __cplusplus
}
#endif
