// Small HBM-bound kernels around the attention kernels: index maps and bias LUTs (offset-aware
// indexing: the explainer's section on offset-aware tiling organises indexing by offset range
// instead of per token pair), per-row dot products with single table rows, and the backward's
// D = rowsum(dO * O).
#include "relpos_device.h"

namespace relpos {

// ----------------------------------------------------------------------------- index maps
__global__ void t5_lut_kernel(const float* __restrict__ beta, int H, int L, int nb, float inv_scale,
                              T5Map m, float* __restrict__ lut) {
  const int n = 2 * L - 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n * H) return;
  const int h = (int)(idx / n);
  const int x = (int)(idx % n);
  const int delta = x - (L - 1);
  const int b = t5_bucket_dev(delta, m);
  lut[idx] = beta[(int64_t)h * nb + b] * inv_scale;
}

hipError_t launch_t5_lut(const float* beta, int H, int L, int nb, float inv_scale, const T5Map& m,
                         float* lut, hipStream_t stream) {
  const int64_t total = (int64_t)(2 * L - 1) * H;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(t5_lut_kernel, dim3(blocks), dim3(256), 0, stream, beta, H, L, nb, inv_scale, m, lut);
  return hipGetLastError();
}

// ALiBi: the bias of offset delta in y units (the kernels scale the LUT by s)
__global__ void alibi_lut_kernel(const float* __restrict__ slopes, int H, int L, float inv_scale,
                                 float* __restrict__ lut) {
  const int n = 2 * L - 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n * H) return;
  const int h = (int)(idx / n);
  const int delta = (int)(idx % n) - (L - 1);
  lut[idx] = -slopes[h] * (float)(delta < 0 ? -delta : delta) * inv_scale;
}

hipError_t launch_alibi_lut(const float* slopes, int H, int L, float inv_scale, float* lut,
                            hipStream_t stream) {
  const int64_t total = (int64_t)(2 * L - 1) * H;
  hipLaunchKernelGGL(alibi_lut_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     slopes, H, L, inv_scale, lut);
  return hipGetLastError();
}

__global__ void index_map_kernel(int mech, int L, int span, int nrel, int txl_off, T5Map m,
                                 int32_t* __restrict__ out_a, int32_t* __restrict__ out_b) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= 2 * L - 1) return;
  const int delta = x - (L - 1);
  int ra;
  if (mech == MECH_T5) ra = t5_bucket_dev(delta, m);
  else if (mech == MECH_ALIBI) ra = delta < 0 ? -delta : delta;   // distinct per offset and sign
  else ra = row_side_row(mech, delta, span, nrel, txl_off);
  out_a[x] = ra;
  if (out_b) out_b[x] = p2c_row(delta, span);
}

hipError_t launch_index_map(int mech, int L, int span, int nrel, int txl_off, const T5Map& m,
                            int32_t* out_a, int32_t* out_b, hipStream_t stream) {
  const int n = 2 * L - 1;
  hipLaunchKernelGGL(index_map_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, mech, L, span,
                     nrel, txl_off, m, out_a, out_b);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- row dots
// 8 lanes per row, 8 elements per lane; results reduced with lane shuffles.
template <typename TX, typename TY>
__global__ void rowdot_kernel(RowDotArgs a) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = gt >> 3;
  const int part = (int)(gt & 7);
  const bool valid = n < a.nrows;
  const int64_t nn = valid ? n : 0;
  const int h = (int)((nn / a.rows_per_head) % a.H);
  const int64_t xoff = a.x_head_stride < 0
                           ? nn * kHeadDim
                           : (int64_t)h * a.x_head_stride + (nn % a.rows_per_head) * kHeadDim;
  float x[8];
  load8((const TX*)a.x + xoff + part * 8, x);
  float acc[2] = {0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (e >= a.ne) break;
    const int row = e == 0 ? a.y_row0 : a.y_row1;
    const TY* y = (const TY*)a.y + (int64_t)h * a.y_head_stride + (int64_t)row * kHeadDim + part * 8;
    float yv[8];
    load8(y, yv);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(x[i], yv[i], s);
    s += __shfl_xor(s, 1, 8);
    s += __shfl_xor(s, 2, 8);
    s += __shfl_xor(s, 4, 8);
    acc[e] = s;
  }
  if (valid && part == 0) {
    for (int e = 0; e < a.ne; ++e) a.out[n * a.ne + e] = acc[e];
  }
}

hipError_t launch_rowdot(const RowDotArgs& a, bool x_fp32, bool y_fp32, hipStream_t stream) {
  const int64_t threads = a.nrows * 8;
  const int blocks = (int)((threads + 255) / 256);
  if (blocks == 0) return hipSuccess;
  if (x_fp32 && y_fp32) hipLaunchKernelGGL((rowdot_kernel<float, float>), dim3(blocks), dim3(256), 0, stream, a);
  else if (x_fp32) hipLaunchKernelGGL((rowdot_kernel<float, uint16_t>), dim3(blocks), dim3(256), 0, stream, a);
  else if (y_fp32) hipLaunchKernelGGL((rowdot_kernel<uint16_t, float>), dim3(blocks), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((rowdot_kernel<uint16_t, uint16_t>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- D = rowsum(dO * O)
template <typename T>
__global__ void dsum_kernel(const T* __restrict__ o, const T* __restrict__ dout, int64_t nrows,
                            float* __restrict__ dsum) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = gt >> 3;
  const int part = (int)(gt & 7);
  const int64_t nn = n < nrows ? n : 0;
  float x[8], y[8];
  load8(o + nn * kHeadDim + part * 8, x);
  load8(dout + nn * kHeadDim + part * 8, y);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf(x[i], y[i], s);
  s += __shfl_xor(s, 1, 8);
  s += __shfl_xor(s, 2, 8);
  s += __shfl_xor(s, 4, 8);
  if (n < nrows && part == 0) dsum[n] = s;
}

hipError_t launch_dsum(const void* o, const void* dout, int64_t nrows, bool fp32, float* dsum,
                       hipStream_t stream) {
  const int64_t threads = nrows * 8;
  const int blocks = (int)((threads + 255) / 256);
  if (blocks == 0) return hipSuccess;
  if (fp32) hipLaunchKernelGGL((dsum_kernel<float>), dim3(blocks), dim3(256), 0, stream, (const float*)o, (const float*)dout, nrows, dsum);
  else hipLaunchKernelGGL((dsum_kernel<uint16_t>), dim3(blocks), dim3(256), 0, stream, (const uint16_t*)o, (const uint16_t*)dout, nrows, dsum);
  return hipGetLastError();
}

}  // namespace relpos
