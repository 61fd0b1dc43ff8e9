// Measurement-only probe: sustained dense bf16 MFMA throughput of the device, so that the
// roofline can be reported against a measured ceiling beside the published one.  Each wave
// runs four independent 32x32x16 accumulation chains on register operands (no memory traffic
// in the loop); the host times the launch with HIP events.
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

}  // namespace

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
