/* Measurement-only entry point, built into librelpos_probe.so beside the attention library.
 * It is not part of the attention path; the benchmark uses it to report the device's sustained
 * dense bf16 MFMA rate next to the published peak. */
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

#ifdef __cplusplus
}
#endif
#endif
