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
// 128 x 128 output tile per workgroup (4 waves, 2 x 2 MFMA blocks of 32 x 32 each), k in steps of 64
// staged through LDS with both operands stored k-contiguous (operands contiguous along m or n
// are transposed on the way in); the next step's global loads are in flight during the
// current step's products.  fp32 operands are split into
// (hi, lo) bf16 planes (three products per MFMA step).  The long-k product (dW) is split over
// k into fixed slices whose fp32 partials are summed in slice order: deterministic.
#include "relpos_device.h"
#include "relpos_kernels.h"

namespace relpos {

namespace {

constexpr int PT = 128;       // output tile (PT x PT per workgroup)
constexpr int SUB = 64;       // staging sub-tile rows
constexpr int PK = 64;        // k step
constexpr int PSTR = PK + 16; // LDS row stride (elements): 40 words, conflict-free with the swizzle
constexpr int NOSPLIT = 1 << 30;

// index i -> (i / split) * s + (i % split) * c, for 0 <= i < 2^31.  The quotient uses a
// multiply-shift divider fixed on the host (q = (umulhi(i, mul) + i) >> shift with
// shift = ceil(log2 split), mul = floor(2^32 (2^shift - split) / split) + 1), exact for every
// i < 2^31 and split <= 2^30: address arithmetic stays off the slow integer-division path.
struct Ix {
  int64_t c, s;
  uint32_t split, mul, shift;
};
Ix mk(int64_t c, int64_t s, uint32_t split) {
  uint32_t l = 0;
  while ((1ull << l) < split) ++l;
  const uint64_t mul = (((1ull << 32) * ((1ull << l) - split)) / split) + 1;
  return Ix{c, s, split, (uint32_t)mul, l};
}
__device__ __forceinline__ int64_t ix(const Ix& m, int i) {
  const uint32_t u = (uint32_t)i;
  const uint32_t q = (__umulhi(u, m.mul) + u) >> m.shift;
  const uint32_t r = u - q * m.split;
  return (int64_t)q * m.s + (int64_t)r * m.c;
}

// An operand in tile coordinates: A as (m, k), B as (n, k).  Exactly one of the two indices
// has unit stride within its split (k_contig: along k), and 8-element groups along it never
// cross a split (splits and extents along it are multiples of 8).
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

// 8 consecutive elements as loaded (no conversion yet)
template <bool F32> struct Raw;
template <> struct Raw<false> { u32x4 v; };
template <> struct Raw<true> { f32x4 a, b; };

template <bool F32>
__device__ __forceinline__ void raw_load(const void* p, int64_t e, Raw<F32>& r) {
  if constexpr (F32) {
    r.a = *(const f32x4*)((const float*)p + e);
    r.b = *(const f32x4*)((const float*)p + e + 4);
  } else {
    r.v = *(const u32x4*)((const uint16_t*)p + e);
  }
}

// element i of a raw group as a float, zero when the group was out of range
template <bool F32>
__device__ __forceinline__ float raw_elem(const Raw<F32>& r, bool ok, int i) {
  float x;
  if constexpr (F32) x = i < 4 ? r.a[i] : r.b[i - 4];
  else x = __uint_as_float((i & 1) ? (r.v[i >> 1] & 0xFFFF0000u) : (r.v[i >> 1] << 16));
  return ok ? x : 0.f;
}

// One thread's share (two groups of 8) of a [64 tile rows] x [64 k] operand sub-tile.
// k-contiguous (KC): row tid / 4, k 16 (tid % 4) + 8 h.  Otherwise: k row 2 (tid / 8) + h,
// tile rows 8 (tid % 8) .. +7 (8 lanes cover 64 contiguous elements of one k row).
// Every load is issued unconditionally (an out-of-range group reads the operand's first 8
// elements and is masked to zero later), so all of a step's loads are in flight together.
template <bool F32, bool KC>
__device__ __forceinline__ void load_stage(const Operand& o, int row0, int nrows, int k0, int kend,
                                           Raw<F32> r[2], bool ok[2]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int row, k;
    if constexpr (KC) { row = row0 + (tid >> 2); k = k0 + (tid & 3) * 16 + 8 * h; }
    else { row = row0 + (tid & 7) * 8; k = k0 + 2 * (tid >> 3) + h; }
    ok[h] = row < nrows && k < kend;
    raw_load<F32>(o.p, ok[h] ? ix(o.row, row) + ix(o.k, k) : 0, r[h]);
  }
}

// Registers -> 64 rows of an LDS tile [NP planes][PT rows][PSTR], k contiguous.  The
// transposing path writes k pairs as 32-bit words; rows are visited in the order i ^ (tid % 8)
// so that the 64 lanes of a store hit distinct banks.  bf16 operands are copied bit for bit
// (their low plane is zero).
template <int NP, bool F32, bool KC>
__device__ __forceinline__ void store_stage(uint16_t* t, const Raw<F32> r[2], const bool ok[2]) {
  const int tid = threadIdx.x;
  constexpr int plane = PT * PSTR;   // t points at row 0 or 64 of a [PT][PSTR] plane
  if constexpr (KC) {
    const int row = tid >> 2, kk = (tid & 3) * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint16_t* dst = t + row * PSTR + kk + 8 * h;
      if constexpr (!F32) {
        u32x4 v = r[h].v;
        if (!ok[h]) v = u32x4{0u, 0u, 0u, 0u};
        *(u32x4*)dst = v;
        if constexpr (NP == 2) *(u32x4*)(dst + plane) = u32x4{0u, 0u, 0u, 0u};
      } else {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = raw_elem<F32>(r[h], ok[h], i);
        Op<NP> v = op_from_f32<NP>(x);
#pragma unroll
        for (int p = 0; p < NP; ++p) *(bf16x8*)(dst + p * plane) = v.p[p];
      }
    }
  } else {
    const int mg = tid & 7, kp = tid >> 3;
    // words[p][u]: plane p of the k pair (k row 2 kp, 2 kp + 1) of tile row 8 mg + u
    uint32_t words[NP][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (!F32) {
        const uint32_t a = __float_as_uint(raw_elem<F32>(r[0], ok[0], u)) >> 16;
        const uint32_t b = __float_as_uint(raw_elem<F32>(r[1], ok[1], u)) & 0xFFFF0000u;
        words[0][u] = a | b;
        if constexpr (NP == 2) words[1][u] = 0u;
      } else {
        uint16_t ha, la, hb, lb;
        split_bf16(raw_elem<F32>(r[0], ok[0], u), ha, la);
        split_bf16(raw_elem<F32>(r[1], ok[1], u), hb, lb);
        words[0][u] = (uint32_t)ha | ((uint32_t)hb << 16);
        if constexpr (NP == 2) words[1][u] = (uint32_t)la | ((uint32_t)lb << 16);
      }
    }
    // words[p][j] <- words[p][j ^ mg] by three conditional butterfly stages
#pragma unroll
    for (int b = 1; b < 8; b <<= 1) {
      const bool sw = (mg & b) != 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u & b) continue;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const uint32_t lo = words[p][u], hi = words[p][u | b];
          words[p][u] = sw ? hi : lo;
          words[p][u | b] = sw ? lo : hi;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = (8 * mg + (j ^ mg)) * PSTR + 2 * kp;
#pragma unroll
      for (int p = 0; p < NP; ++p) *(uint32_t*)(t + p * plane + e) = words[p][j];
    }
  }
}

// AF / BF: operand A / B is fp32 (else bf16); AKC / BKC: k-contiguous.  fp32 anywhere means
// two bf16 planes (hi, lo) per operand and three products per step.
template <bool AF, bool AKC, bool BF, bool BKC>
__global__ __launch_bounds__(256) void proj_gemm_kernel(GemmArgs g) {
  constexpr int NP = (AF || BF) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t stage_lds[2 * NP * PT * PSTR];
  uint16_t* as = stage_lds;
  uint16_t* bs = stage_lds + NP * PT * PSTR;
  const int tiles_n = (g.N + PT - 1) / PT;
  const int tiles = ((g.M + PT - 1) / PT) * tiles_n;
  // consecutive ids (the n tiles of one m tile, which share A rows) run on one XCD's L2
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = id / tiles;
  const int tile = id % tiles;
  const int m0 = (tile / tiles_n) * PT, n0 = (tile % tiles_n) * PT;
  const int kper = ((g.K + g.kslices - 1) / g.kslices + PK - 1) / PK * PK;
  const int kb = slice * kper, ke = min(g.K, kb + kper);
  const int w = wave_index(), lane = threadIdx.x & 63, l32 = lane & 31, kh = lane >> 5;
  const int wm = w >> 1, wn = w & 1;   // wave block: rows 64 wm.., cols 64 wn.. (2 x 2 MFMA blocks)
  f32x16 acc[2][2] = {};
  Raw<AF> ra[2][2];
  Raw<BF> rb[2][2];
  bool oka[2][2], okb[2][2];
  if (kb < ke) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      load_stage<AF, AKC>(g.a, m0 + SUB * u, g.M, kb, ke, ra[u], oka[u]);
      load_stage<BF, BKC>(g.b, n0 + SUB * u, g.N, kb, ke, rb[u], okb[u]);
    }
  }
  for (int k0 = kb; k0 < ke; k0 += PK) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      store_stage<NP, AF, AKC>(as + SUB * u * PSTR, ra[u], oka[u]);
      store_stage<NP, BF, BKC>(bs + SUB * u * PSTR, rb[u], okb[u]);
    }
    __syncthreads();
    if (k0 + PK < ke) {   // next step's loads fly while this step's products run
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        load_stage<AF, AKC>(g.a, m0 + SUB * u, g.M, k0 + PK, ke, ra[u], oka[u]);
        load_stage<BF, BKC>(g.b, n0 + SUB * u, g.N, k0 + PK, ke, rb[u], okb[u]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < PK; kk += 16) {
      Op<NP> ao[2], bo[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        ao[b] = op_from_lds<NP>(as, PT * PSTR, (wm * 64 + 32 * b + l32) * PSTR + kk + 8 * kh);
        bo[b] = op_from_lds<NP>(bs, PT * PSTR, (wn * 64 + 32 * b + l32) * PSTR + kk + 8 * kh);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma<NP>(acc[i][j], ao[i], bo[j]);   // n on the lanes
    }
  }
  // Epilogue through LDS, one 32-column half of each wave's 64 x 64 block at a time: the
  // accumulators (acc[i][j] register r: m = 64 wm + 32 i + 8 (r / 4) + 4 kh + r % 4,
  // n = 64 wn + 32 j + l32) go to a wave-private [64][CSTR] fp32 patch, and each lane then
  // writes 8 consecutive n of one row with vector stores (C is contiguous along n in 8-groups).
  constexpr int CSTR = 40;
  static_assert(4 * 64 * CSTR * 4 <= 2 * PT * PSTR * 2, "C patch fits the A / B staging area");
  float* patch = reinterpret_cast<float*>(as) + w * 64 * CSTR;   // as and bs are contiguous
  float* cbase = g.c16 ? nullptr : g.c + (int64_t)slice * g.c_slice;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    __syncthreads();   // previous readers of the staging area are done
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        patch[(32 * i + 8 * (r >> 2) + 4 * kh + (r & 3)) * CSTR + l32] = acc[i][j][r];
    __syncthreads();
    const int q = lane & 3, n = n0 + wn * 64 + 32 * j + 8 * q;
    if (n >= g.N) continue;
    const int64_t on = ix(g.cn, n);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = (lane >> 2) + 16 * t, m = m0 + wm * 64 + row;
      if (m >= g.M) continue;
      const float* src = patch + row * CSTR + 8 * q;
      const f32x4 lo = *(const f32x4*)src, hi = *(const f32x4*)(src + 4);
      const int64_t o = ix(g.cm, m) + on;
      if (g.c16) {
        u32x4 v;
        v[0] = pack_bf16x2(lo[0], lo[1]);
        v[1] = pack_bf16x2(lo[2], lo[3]);
        v[2] = pack_bf16x2(hi[0], hi[1]);
        v[3] = pack_bf16x2(hi[2], hi[3]);
        *(u32x4*)(g.c16 + o) = v;
      } else {
        *(f32x4*)(cbase + o) = lo;
        *(f32x4*)(cbase + o + 4) = hi;
      }
    }
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

template <bool AF, bool AKC, bool BF, bool BKC>
void launch_gemm(const GemmArgs& g, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((proj_gemm_kernel<AF, AKC, BF, BKC>), grid, dim3(256), 0, st, g);
}

// The three products: forward (A k-contiguous, B not; one dtype), dX (both k-contiguous, A
// fp32) and dW (neither, B fp32).
hipError_t run_gemm(GemmArgs g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int tiles = ((g.M + PT - 1) / PT) * ((g.N + PT - 1) / PT);
  const dim3 grid((unsigned)(tiles * g.kslices));
  const bool af = g.a.fp32, ak = g.a.k_contig, bf = g.b.fp32, bk = g.b.k_contig;
  if (!af && ak && !bf && !bk) launch_gemm<false, true, false, false>(g, grid, st);
  else if (af && ak && bf && !bk) launch_gemm<true, true, true, false>(g, grid, st);
  else if (af && ak && !bf && bk) launch_gemm<true, true, false, true>(g, grid, st);
  else if (af && ak && bf && bk) launch_gemm<true, true, true, true>(g, grid, st);
  else if (!af && !ak && bf && !bk) launch_gemm<false, false, true, false>(g, grid, st);
  else if (af && !ak && bf && !bk) launch_gemm<true, false, true, false>(g, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

// rel [H, N, d] (bf16 or fp32) = X [N, F] . W [F, H d]
hipError_t launch_project_fwd(const void* X, const void* W, void* rel, int N, int F, int H, int d,
                              bool fp32, hipStream_t st) {
  GemmArgs g{};
  g.a = Operand{X, mk(F, 0, NOSPLIT), mk(1, 0, NOSPLIT), fp32, true};        // X[n_row][f]
  g.b = Operand{W, mk(1, 0, NOSPLIT), mk(H * d, 0, NOSPLIT), fp32, false};   // W[f][col], n = col
  if (fp32) g.c = (float*)rel; else g.c16 = (uint16_t*)rel;
  g.cm = mk(d, 0, NOSPLIT);                       // rel[col / d][n_row][col % d]
  g.cn = mk(1, (int64_t)N * d, d);
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
    g.a = Operand{drel, mk(d, 0, NOSPLIT), mk(1, (int64_t)N * d, d), true, true};   // m = n_row, k = col
    g.b = Operand{W, mk(H * d, 0, NOSPLIT), mk(1, 0, NOSPLIT), fp32, true};          // n = f, k = col
    g.c = dX;
    g.cm = mk(F, 0, NOSPLIT);
    g.cn = mk(1, 0, NOSPLIT);
    g.M = N; g.N = F; g.K = H * d; g.kslices = 1;
    e = run_gemm(g, st);
    if (e != hipSuccess) return e;
  }
  if (dW) {
    GemmArgs g{};
    g.a = Operand{X, mk(1, 0, NOSPLIT), mk(F, 0, NOSPLIT), fp32, false};             // m = f, k = n_row
    g.b = Operand{drel, mk(1, (int64_t)N * d, d), mk(d, 0, NOSPLIT), true, false};   // n = col, k = n_row
    g.c = kslices > 1 ? partials : dW;
    g.cm = mk(H * d, 0, NOSPLIT);
    g.cn = mk(1, 0, NOSPLIT);
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
