// Measurement-only probes: sustained dense bf16 MFMA throughput of the device, so that the
// roofline can be reported against a measured ceiling beside the published one, and the
// sustained rates of the two vector-ALU operations every softmax weight needs (the base-2
// exponential and the fp32 fused multiply-add), which bound the passes whose per-score vector
// work outweighs their matrix work.  Each wave runs independent chains on register operands
// (no memory traffic in the loop); the host times the launch with HIP events.
#include <hip/hip_runtime.h>

#include "relpos_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((threadIdx.x + 3 * i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// kind 0: v_exp_f32 (2^x); kind 1: v_fma_f32.  Eight independent chains per lane, so the
// loop is bound by issue, not by the latency of one chain.  The exponential chain iterates
// x <- 2^-x (the negation is a free source modifier), which converges to its fixed point near
// 0.64, so every operand stays an ordinary normal number.
template <int KIND>
__global__ __launch_bounds__(256) void valu_probe_kernel(int iters, float* out) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 1.0f + 0.01f * (float)((threadIdx.x + i) & 15);
  const float m = 0.999f, c = 0.0005f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (KIND == 0) x[i] = __builtin_amdgcn_exp2f(-x[i]);
        else x[i] = __builtin_fmaf(x[i], m, c);
      }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Matrix / vector overlap.  One unit of work is 4 bf16 MFMAs (32x32x16, four independent
// chains) or 8 exponentials plus 24 fp32 FMAs (eight independent chains), about the vector work
// a softmax step puts beside that many MFMAs.  MODE 0: every wave runs `iters` matrix units;
// MODE 1: `iters` vector units; MODE 2: every wave interleaves `iters` units of each (overlap
// inside a wave); MODE 3: even workgroups run the matrix units and odd ones the vector units
// (overlap between the waves that share a SIMD).  Comparing the times of MODE 2 (or MODE 3 at
// twice the workgroups) with the sum and the maximum of MODE 0 and MODE 1 shows how much of the
// vector work hides under the matrix work.
template <int MODE>
__device__ __forceinline__ void overlap_body(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((threadIdx.x + 3 * i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 1.0f + 0.01f * (float)((threadIdx.x + i) & 15);
  // (MODE 3: the wave's kind is uniform across the wave, threadIdx.x / 256)
  const bool do_m = MODE == 0 || MODE == 2 || (MODE == 3 && threadIdx.x < 256);
  const bool do_v = MODE == 1 || MODE == 2 || (MODE == 3 && threadIdx.x >= 256);
  const float m = 0.999f, c = 0.0005f;
  for (int it = 0; it < iters; ++it) {
    if (do_m) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    if (do_v) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = __builtin_amdgcn_exp2f(-x[i]);
        x[i] = __builtin_fmaf(x[i], m, c);
        x[i] = __builtin_fmaf(x[i], m, c);
        x[i] = __builtin_fmaf(x[i], m, c);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int MODE>
__global__ __launch_bounds__(256, 4) void overlap_probe_kernel(int iters, float* out) {
  overlap_body<MODE>(iters, out);
}

__global__ __launch_bounds__(512, 2) void overlap_probe_split_kernel(int iters, float* out) {
  overlap_body<3>(iters, out);
}

template <typename F>
int time_launch(hipStream_t st, F launch, float* ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -4;
  if (hipEventCreate(&e1) != hipSuccess) { hipEventDestroy(e0); return -4; }
  launch();   // untimed
  hipEventRecord(e0, st);
  launch();
  hipEventRecord(e1, st);
  const hipError_t err = hipEventSynchronize(e1);
  *ms = 0.f;
  if (err == hipSuccess) hipEventElapsedTime(ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (err != hipSuccess || hipGetLastError() != hipSuccess || *ms <= 0.f) return -4;
  return 0;
}

}  // namespace

extern "C" int relpos_probe_valu(int kind, int iters, int blocks, float* out, double* gops,
                                 void* stream) {
  if ((kind != 0 && kind != 1) || iters <= 0 || blocks <= 0 || out == nullptr || gops == nullptr)
    return -1;
  hipStream_t st = (hipStream_t)stream;
  float ms = 0.f;
  const int rc = time_launch(st, [&] {
    if (kind == 0) hipLaunchKernelGGL(valu_probe_kernel<0>, dim3(blocks), dim3(256), 0, st, iters, out);
    else hipLaunchKernelGGL(valu_probe_kernel<1>, dim3(blocks), dim3(256), 0, st, iters, out);
  }, &ms);
  if (rc != 0) return rc;
  const double ops = (double)blocks * 256.0 * (double)iters * 32.0;
  *gops = ops / ((double)ms * 1e-3) / 1e9;
  return 0;
}

extern "C" int relpos_probe_overlap(int mode, int iters, int blocks, float* out, double* ms_out,
                                    void* stream) {
  if (mode < 0 || mode > 3 || iters <= 0 || blocks <= 0 || out == nullptr || ms_out == nullptr)
    return -1;
  hipStream_t st = (hipStream_t)stream;
  float ms = 0.f;
  const int rc = time_launch(st, [&] {
    switch (mode) {
      case 0: hipLaunchKernelGGL(overlap_probe_kernel<0>, dim3(blocks), dim3(256), 0, st, iters, out); break;
      case 1: hipLaunchKernelGGL(overlap_probe_kernel<1>, dim3(blocks), dim3(256), 0, st, iters, out); break;
      case 2: hipLaunchKernelGGL(overlap_probe_kernel<2>, dim3(blocks), dim3(256), 0, st, iters, out); break;
      default: hipLaunchKernelGGL(overlap_probe_split_kernel, dim3(blocks), dim3(512), 0, st, iters, out); break;
    }
  }, &ms);
  if (rc != 0) return rc;
  *ms_out = ms;
  return 0;
}

extern "C" int relpos_probe_mfma_bf16(int iters, int blocks, float* out, double* tflops,
                                      void* stream) {
  if (iters <= 0 || blocks <= 0 || out == nullptr || tflops == nullptr) return -1;
  hipStream_t st = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -4;
  if (hipEventCreate(&e1) != hipSuccess) { hipEventDestroy(e0); return -4; }
  // one untimed launch, then the timed one
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, st, iters, out);
  hipEventRecord(e0, st);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, st, iters, out);
  hipEventRecord(e1, st);
  const hipError_t err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (err == hipSuccess) hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (err != hipSuccess || hipGetLastError() != hipSuccess || ms <= 0.f) return -4;
  const double flops = (double)blocks * 4.0 /* waves */ * (double)iters * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
  *tflops = flops / ((double)ms * 1e-3) / 1e12;
  return 0;
}
