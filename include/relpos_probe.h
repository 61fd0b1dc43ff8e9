/* Measurement-only entry points, built into librelpos_probe.so beside the attention library.
 * They are not part of the attention path; the benchmark uses them to report the device's
 * sustained dense bf16 MFMA rate next to the published peak, and the sustained vector-ALU rates
 * of the base-2 exponential and the fp32 fused multiply-add that bound the softmax work. */
#ifndef RELPOS_PROBE_H
#define RELPOS_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Runs `blocks` workgroups of 256 threads, each wave issuing 4 * iters back-to-back
 * v_mfma_f32_32x32x16_bf16 on register operands, and writes the sustained rate of the timed
 * launch (TFLOP/s, 2 flops per multiply-add) to *tflops.  `out` is device memory of
 * blocks * 256 floats that receives the accumulator sums (so the work is not removed).
 * Blocks the calling thread until the launch completes.  Returns 0, -1 for a bad argument,
 * -4 for a HIP error. */
int relpos_probe_mfma_bf16(int iters, int blocks, float* out, double* tflops, void* stream);

/* Runs `blocks` workgroups of 256 threads, each lane issuing 32 * iters vector operations of
 * one kind in eight independent chains: kind 0 = v_exp_f32 (2^x), kind 1 = v_fma_f32.  Writes
 * the sustained rate of the timed launch in giga lane-operations per second to *gops.  `out`
 * as for relpos_probe_mfma_bf16.  Blocks the calling thread until the launch completes.
 * Returns 0, -1 for a bad argument, -4 for a HIP error. */
int relpos_probe_valu(int kind, int iters, int blocks, float* out, double* gops, void* stream);

/* Matrix / vector overlap: `blocks` workgroups of 256 threads run `iters` units of work, a
 * matrix unit being 4 back-to-back v_mfma_f32_32x32x16_bf16 and a vector unit 8 v_exp_f32 and
 * 24 v_fma_f32.  mode 0: matrix units only; 1: vector units only; 2: every wave runs both,
 * interleaved; 3: workgroups of 512 threads (`out` then holds blocks * 512 floats) whose waves
 * 0-3 run matrix units and waves 4-7 vector units, so every SIMD holds a wave of each kind.
 * Writes the timed launch's duration in milliseconds to *ms.  `out` as for
 * relpos_probe_mfma_bf16 otherwise.  Blocks the
 * calling thread until the launch completes.  Returns 0, -1 for a bad argument, -4 for a HIP
 * error. */
int relpos_probe_overlap(int mode, int iters, int blocks, float* out, double* ms, void* stream);

#ifdef __cplusplus
}
#endif
#endif
