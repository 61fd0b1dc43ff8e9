// Relation-table projections on MFMA: the prologue that turns a position basis into the
// relation table the attention kernels read (T-XL r = R W_r, DeBERTa Kr = P W_r^k and
// Qr = P W_r^q) and the epilogue that takes the table gradient back to dW and dX.  The
// explainer's section on reusing query-key relation products treats these decomposable
// "bias vector x position embedding" terms; the projections are the mechanisms' own
// definitions.  All three products are one GEMM over strided, head-split operands:
//
//   C(m, n) = sum_k A(m, k) B(n, k),   each index i of an operand at (i / split) s + (i % split) c
//
// (the head split turns the [H, N, d] table into the [N, H d] matrix the products need).
// 64 x 64 output tile per workgroup (4 waves, one 32 x 32 MFMA block each), k in steps of 32
// staged through LDS with both operands stored k-contiguous.  fp32 operands are split into
// (hi, lo) bf16 planes (three products per MFMA step).  The long-k product (dW) is split over
// k into fixed slices whose fp32 partials are summed in slice order: deterministic.
#include "relpos_device.h"
#include "relpos_kernels.h"

namespace relpos {

namespace {

constexpr int PT = 64;        // output tile
constexpr int PK = 32;        // k step
constexpr int PSTR = PK + 8;  // LDS row stride (elements)
constexpr int NOSPLIT = 1 << 30;

// index i -> (i / split) * s + (i % split) * c
struct Ix {
  int64_t c, s;
  int split;
};
__device__ __forceinline__ int64_t ix(const Ix& m, int i) {
  return (int64_t)(i / m.split) * m.s + (int64_t)(i % m.split) * m.c;
}

// An operand in tile coordinates: A as (m, k), B as (n, k).  Exactly one of the two indices
// has unit stride within its split (k_contig: along k), and 8-element groups along it never
// cross a split (splits and tile extents along it are multiples of 8).
struct Operand {
  const void* p;
  Ix row, k;
  bool fp32;
  bool k_contig;
};

struct GemmArgs {
  Operand a, b;            // A(m, k), B(n, k)
  float* c;                // C(m, n), fp32 ...
  uint16_t* c16;           // ... or bf16
  Ix cm, cn;
  int M, N, K;
  int kslices;             // k split (fp32 partials at c + slice * c_slice)
  int64_t c_slice;
};

// 8 elements from element offset e, consecutive in memory, as floats
__device__ __forceinline__ void load8v(const Operand& o, int64_t e, float x[8]) {
  if (o.fp32) load8((const float*)o.p + e, x);
  else load8((const uint16_t*)o.p + e, x);
}

// Stage a [64 tile rows] x [32 k] tile into NP planes of [64][PSTR] bf16, k contiguous.
template <int NP>
__device__ __forceinline__ void stage_tile(uint16_t* t, const Operand& o, int row0, int nrows,
                                           int k0, int kend) {
  const int tid = threadIdx.x;
  const int plane = PT * PSTR;
  float x[8];
  if (o.k_contig) {
    // thread -> (row, 8 consecutive k)
    const int row = tid >> 2, kk = (tid & 3) * 8;
    if (row0 + row < nrows && k0 + kk < kend) {
      load8v(o, ix(o.row, row0 + row) + ix(o.k, k0 + kk), x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    Op<NP> v = op_from_f32<NP>(x);
#pragma unroll
    for (int p = 0; p < NP; ++p) *(bf16x8*)(t + p * plane + row * PSTR + kk) = v.p[p];
  } else {
    // thread -> (k, 8 consecutive rows), scattered into the k-contiguous layout
    const int kk = tid >> 3, row = (tid & 7) * 8;
    if (k0 + kk < kend && row0 + row < nrows) {
      load8v(o, ix(o.row, row0 + row) + ix(o.k, k0 + kk), x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t h, l;
      split_bf16(x[i], h, l);
      t[(row + i) * PSTR + kk] = h;
      if constexpr (NP == 2) t[plane + (row + i) * PSTR + kk] = l;
    }
  }
}

template <int NP>
__global__ __launch_bounds__(256) void proj_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t as[NP * PT * PSTR];
  __shared__ __attribute__((aligned(16))) uint16_t bs[NP * PT * PSTR];
  const int tiles_n = (g.N + PT - 1) / PT;
  const int tiles = ((g.M + PT - 1) / PT) * tiles_n;
  const int slice = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int m0 = (tile / tiles_n) * PT, n0 = (tile % tiles_n) * PT;
  const int kper = ((g.K + g.kslices - 1) / g.kslices + PK - 1) / PK * PK;
  const int kb = slice * kper, ke = min(g.K, kb + kper);
  const int w = wave_index(), lane = threadIdx.x & 63, l32 = lane & 31, kh = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  f32x16 acc = {};
  for (int k0 = kb; k0 < ke; k0 += PK) {
    __syncthreads();
    stage_tile<NP>(as, g.a, m0, g.M, k0, ke);
    stage_tile<NP>(bs, g.b, n0, g.N, k0, ke);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < PK; kk += 16) {
      Op<NP> ao = op_from_lds<NP>(as, PT * PSTR, (wm * 32 + l32) * PSTR + kk + 8 * kh);
      Op<NP> bo = op_from_lds<NP>(bs, PT * PSTR, (wn * 32 + l32) * PSTR + kk + 8 * kh);
      mma<NP>(acc, ao, bo);   // acc[m][n], n on the lanes
    }
  }
  // acc register r: m = wm 32 + 8 (r / 4) + 4 kh + r % 4, n = wn 32 + l32
  const int n = n0 + wn * 32 + l32;
  if (n >= g.N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wm * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
    if (m >= g.M) continue;
    const int64_t o = ix(g.cm, m) + ix(g.cn, n);
    if (g.c16) g.c16[o] = f2bf_bits(acc[r]);
    else g.c[(int64_t)slice * g.c_slice + o] = acc[r];
  }
}

// out[i] = sum_{s < S} part[s * n + i] in slice order
__global__ void slice_sum_kernel(const float* __restrict__ part, int S, int64_t n,
                                 float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int s = 0; s < S; ++s) acc += part[(int64_t)s * n + i];
  out[i] = acc;
}

hipError_t run_gemm(GemmArgs g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int tiles = ((g.M + PT - 1) / PT) * ((g.N + PT - 1) / PT);
  const dim3 grid((unsigned)(tiles * g.kslices));
  if (g.a.fp32 || g.b.fp32) hipLaunchKernelGGL(proj_gemm_kernel<2>, grid, dim3(256), 0, st, g);
  else hipLaunchKernelGGL(proj_gemm_kernel<1>, grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace

// rel [H, N, d] (bf16 or fp32) = X [N, F] . W [F, H d]
hipError_t launch_project_fwd(const void* X, const void* W, void* rel, int N, int F, int H, int d,
                              bool fp32, hipStream_t st) {
  GemmArgs g{};
  g.a = Operand{X, Ix{F, 0, NOSPLIT}, Ix{1, 0, NOSPLIT}, fp32, true};        // X[n_row][f]
  g.b = Operand{W, Ix{1, 0, NOSPLIT}, Ix{H * d, 0, NOSPLIT}, fp32, false};   // W[f][col], n = col
  if (fp32) g.c = (float*)rel; else g.c16 = (uint16_t*)rel;
  g.cm = Ix{d, 0, NOSPLIT};                       // rel[col / d][n_row][col % d]
  g.cn = Ix{1, (int64_t)N * d, d};
  g.M = N; g.N = H * d; g.K = F; g.kslices = 1;
  return run_gemm(g, st);
}

// dX [N, F] = dY . W^T and dW [F, H d] = X^T . dY, dY(n_row, col) = drel[col / d][n_row][col % d]
hipError_t launch_project_bwd(const void* X, const void* W, const float* drel, float* dX, float* dW,
                              float* partials, int kslices, int N, int F, int H, int d, bool fp32,
                              hipStream_t st) {
  hipError_t e = hipSuccess;
  if (dX) {
    GemmArgs g{};
    g.a = Operand{drel, Ix{d, 0, NOSPLIT}, Ix{1, (int64_t)N * d, d}, true, true};   // m = n_row, k = col
    g.b = Operand{W, Ix{H * d, 0, NOSPLIT}, Ix{1, 0, NOSPLIT}, fp32, true};          // n = f, k = col
    g.c = dX;
    g.cm = Ix{F, 0, NOSPLIT};
    g.cn = Ix{1, 0, NOSPLIT};
    g.M = N; g.N = F; g.K = H * d; g.kslices = 1;
    e = run_gemm(g, st);
    if (e != hipSuccess) return e;
  }
  if (dW) {
    GemmArgs g{};
    g.a = Operand{X, Ix{1, 0, NOSPLIT}, Ix{F, 0, NOSPLIT}, fp32, false};             // m = f, k = n_row
    g.b = Operand{drel, Ix{1, (int64_t)N * d, d}, Ix{d, 0, NOSPLIT}, true, false};   // n = col, k = n_row
    g.c = kslices > 1 ? partials : dW;
    g.cm = Ix{H * d, 0, NOSPLIT};
    g.cn = Ix{1, 0, NOSPLIT};
    g.M = F; g.N = H * d; g.K = N; g.kslices = kslices; g.c_slice = (int64_t)F * H * d;
    e = run_gemm(g, st);
    if (e != hipSuccess || kslices <= 1) return e;
    const int64_t n = (int64_t)F * H * d;
    hipLaunchKernelGGL(slice_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       partials, kslices, n, dW);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace relpos
