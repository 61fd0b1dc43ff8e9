// Second pass of offset-based gradient sharding (zicq.com explainer, section on offset-based
// gradient sharding: aggregate locally first, then merge): every table-gradient element sums
// the per-workgroup partials in ascending owner order, and reductions over offsets use a fixed
// tree, so the result is bitwise reproducible.  Outputs are overwritten.
#include "relpos_tile.h"

namespace relpos {

// Sum of the partials of owners m = 0 .. n - 1 (owner m at p + slot(m) * stride) with 8 loads in
// flight: running sum j takes the owners m with m % 8 == j; the eight sums are then added in a
// fixed tree.  Deterministic for a given n.
template <typename F>
__device__ __forceinline__ float strided_sum(const float* __restrict__ p, int64_t stride, int n,
                                             F slot) {
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int o = 0;
  for (; o + 8 <= n; o += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] += p[slot(o + j) * stride];
  }
  for (int j = 0; o + j < n; ++j) a[j] += p[slot(o + j) * stride];
  return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// out[h nelem + e] = scale * sum over the owners of head h of part[slot * stride + e].  The
// owners of one output form `runs` runs of run_len consecutive slots, run r starting at slot
// h run_len + r run_stride (one run over every slot when the table is shared).  64 elements per
// workgroup (blockIdx.y = head); the owners, in ascending order o = 0 .. runs run_len - 1, are
// split over four thread groups (group g takes o = g mod 4, each with eight loads in flight),
// whose sums are added in a fixed tree: ((g0 + g1) + (g2 + g3)).
__global__ __launch_bounds__(256) void agg_rows_kernel(const float* __restrict__ part,
                                                       int64_t stride, int runs, int run_len,
                                                       int64_t run_stride, int64_t nelem,
                                                       float scale, float* __restrict__ out) {
  __shared__ float sh[4][64];
  const int g = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int h = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * 64 + l;
  const int nown = runs * run_len;
  float acc = 0.f;
  if (e < nelem && g < nown) {
    const int n = (nown - g + 3) / 4;   // owners g, g + 4, ...
    const int64_t base = (int64_t)h * run_len;
    acc = strided_sum(part + e, stride, n, [=](int m) -> int64_t {
      const int o = g + 4 * m, r = o / run_len;
      return base + (int64_t)r * run_stride + (o - r * run_len);
    });
  }
  sh[g][l] = acc;
  __syncthreads();
  if (g == 0 && e < nelem)
    out[(int64_t)h * nelem + e] = ((sh[0][l] + sh[1][l]) + (sh[2][l] + sh[3][l])) * scale;
}

__device__ __forceinline__ int floordiv32(int a) { return a >= 0 ? a / 32 : -((31 - a) / 32); }

// diag[h][delta + L - 1] = sum over (b, block, wave) of the per-offset dS sums.  The query-side
// pass writes one partial row per wave: wave w of the workgroup at block blk (position p, blk = p
// or, under a causal mask, nb - 1 - p) at slot ((b H + h) nb + p) NWAVE + w, offset delta at
// index delta - (32 u - L - 64) - diag_xoff(blk) with u = 4 blk + w.  One workgroup per (head,
// 64 consecutive offsets): only the wave rows u that can hold one of them are visited, in
// ascending (b, u) order split into consecutive parts, one per thread group of 64 (four groups,
// or sixteen for window-compact rows; 16 loads in flight; the address advances by a constant
// per step within a block); the group sums are then added in group order.
template <bool REV, bool COMPACT>
__global__ __launch_bounds__(COMPACT ? 1024 : 256) void agg_diag_kernel(
    const float* __restrict__ pdiag, int B, int H, int L, int nb, int wl, int wr,
    float* __restrict__ diag) {
  // thread groups of 64 (one per offset); compact rows: few workgroups hold data, so 16 groups
  constexpr int NG = COMPACT ? 16 : 4;
  __shared__ float sh[NG][64];
  const int t = threadIdx.x, j = t & 63, g = t >> 6;
  const int n = 2 * L - 1, nch = (n + 63) / 64;
  // heads vary fastest along the grid: the workgroups that land on one CU then hold chunks
  // spread over the offset range (the owner count of a chunk falls off away from offset 0), and
  // each XCD (workgroups go to the XCDs in turn) reads the partials of fewer heads
  const int h = blockIdx.x % H, c0 = 64 * (blockIdx.x / H);
  const bool valid = c0 + j < n;
  const int ndg = diag_width(L, wl, wr);
  // lane offset delta = c0 + j - (L - 1) sits at x = lim - xs(u) of wave row u, with
  // xs(u) = 32 u + diag_xoff(blk)
  const int a0 = c0 - (L - 1) + L + 64, lim = a0 + j;
  int u_lo, u_hi;
  if (!COMPACT) {   // x = lim - 32 u in [0, ndg)
    u_lo = max(0, floordiv32(a0 - ndg) + 1);
    u_hi = min(NWAVE * nb - 1, floordiv32(a0 + 63));
  } else {          // every block sweeps the offsets near the diagonal; none holds the rest
    const int64_t d0 = c0 - (L - 1);
    const bool any = d0 + 63 >= -((int64_t)wr + 320) && d0 <= (int64_t)wl + 320;
    u_lo = 0;
    u_hi = any ? NWAVE * nb - 1 : -1;
  }
  const int nu = max(0, u_hi - u_lo + 1);
  const int nq = B * nu, per = (nq + NG - 1) / NG;
  const int qa = min(nq, g * per), qb = min(nq, qa + per);
  auto xs_of = [&](int uu) { return 32 * uu + (COMPACT ? diag_xoff(L, wl, wr, 128 * (uu >> 2)) : 0); };
  auto elem_of = [&](int bb, int uu) -> int64_t {
    const int64_t own0 = ((int64_t)bb * H + h) * nb;
    const int64_t slot = REV ? (own0 + nb - 1 - (uu >> 2)) * NWAVE + (uu & 3) : own0 * NWAVE + uu;
    return slot * ndg + (lim - xs_of(uu));
  };
  int b = nu > 0 ? qa / nu : 0, u = u_lo + (nu > 0 ? qa - b * nu : 0);
  const float* ptr = pdiag + (qa < qb ? elem_of(b, u) : 0);
  int xs = xs_of(u);
  // the next wave row of the same block is the next slot (x 32 lower); full-sweep rows continue
  // into the next block the same way (under a causal mask its first wave row lies 7 slots lower);
  // compact rows restart at the block's own offset
  const int64_t inc = (int64_t)ndg - 32, inc_rev = -(int64_t)7 * ndg - 32;
  constexpr int G = 16;
  float acc = 0.f;
  for (int q0 = qa; q0 < qb; q0 += G) {
    float ld[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int x = lim - xs;
      ld[k] = (valid && q0 + k < qb && x >= 0 && x < ndg) ? *ptr : 0.f;
      if (u == u_hi) {
        ++b;
        u = u_lo;
        if (b < B) {
          ptr = pdiag + elem_of(b, u);
          xs = xs_of(u);
        }
      } else if (COMPACT && (u & 3) == 3) {
        ++u;
        ptr = pdiag + elem_of(b, u);
        xs = xs_of(u);
      } else {
        ptr += (REV && (u & 3) == 3) ? inc_rev : inc;
        ++u;
        xs += 32;
      }
    }
#pragma unroll
    for (int k = 0; k < G; ++k) acc += ld[k];
  }
  sh[g][j] = acc;
  __syncthreads();
  if (t < 64 && valid) {
    float sum = sh[0][t];
#pragma unroll
    for (int i = 1; i < NG; ++i) sum += sh[i][t];
    diag[(int64_t)h * n + c0 + t] = sum;
  }
}

// T-XL dr[h][row][d] = s (sum_{b, key block} part[own][x][d] + v_h[d] diag_h[delta]).
// The partials come from the dK/dV pass: owner (slice, p) holds offset delta at row
// x = delta + 128 p + 192 - rbase(p), where rbase = 0 for a full sweep and, with a two-sided
// window, the first row of the owner's sweep (its first 64-row step + 65).  One workgroup
// per (head, 64 consecutive offsets): for every owner the 64 rows it holds for those offsets
// are one contiguous 16 KB block, read whole and added in a fixed owner order.  The slices are
// processed in groups [s0, s0 + ns) of the nslices slices (slot i nb + p for slice s0 + i),
// launched for the heads with a slice in the group only: a head's first group (the one holding
// its slice h) starts from zero, later ones from the raw sums already in dr, and its last group
// applies v . diag and s.  With `shared`, one table serves every head: a single "head" of
// workgroups sums the slices of every head, the call flags `first` / `last` mark its first and
// last group, and the last group's diagonal term is sum_h v_h . diag_h (heads in order).
__global__ __launch_bounds__(256) void agg_txl_dr_kernel(const float* __restrict__ prow,
                                                         const float* __restrict__ diag,
                                                         const float* __restrict__ v, int H,
                                                         int L, int nb, int nrt, int wl, int wr,
                                                         int nrel, int off, float s, int s0,
                                                         int ns, int nslices, int first, int last,
                                                         int shared, float* __restrict__ dr) {
  const int nch = (nrel + 63) / 64;
  // heads vary fastest along the grid, as in agg_diag_kernel.  The grid holds only the heads
  // with a slice in this group, hb = 0 .. HG - 1 for head (s0 + hb) mod H (one when shared), so
  // a group of a few heads still spreads its work over every XCD.
  const int HG = gridDim.x / nch;
  const int hb = blockIdx.x % HG, row0 = 64 * (blockIdx.x / HG);
  const int h = shared ? 0 : (s0 + hb) % H;
  const int t = threadIdx.x;
  const int delta0 = row0 - off;
  // this head's slices in the group: local i = i0, i0 + H, ... (every slice when shared)
  const int hstep = shared ? 1 : H;
  const int i0 = shared ? 0 : ((h - s0) % H + H) % H;
  const int nh = i0 < ns ? (ns - i0 + hstep - 1) / hstep : 0;
  // head h's slices are h, h + H, ...: this group holds its first one when s0 <= h, and its last
  // one when the next slice of h after the group's lies past the end
  const bool head_first = shared ? first != 0 : h >= s0;
  const bool head_last = shared ? last != 0 : s0 + i0 + nh * H >= nslices;
  f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
  if (!head_first) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 4 * t + 1024 * k, row = row0 + (e >> 6);
      if (row < nrel) acc[k] = *(const f32x4*)(dr + ((int64_t)h * nrel + row) * kHeadDim + (e & 63));
    }
  }
  // owner p holds these 64 offsets at its partial rows x0(p) .. x0(p) + 63; x0 does not decrease
  // with p (with a two-sided window it is constant once 128 p > wr), so the owners that hold any
  // of them form one range [p_lo, p_hi], the same for every slice
  auto x0of = [&](int p) {
    const int rbase = (wl >= 0 && wr >= 0) ? (max(0, 128 * p - wr) / 64) * 64 + 65 : 0;
    return delta0 + 128 * p + 192 - rbase;
  };
  int lo = 0, hi = nb;   // p_lo: the first p with x0 + 63 >= 0
  while (lo < hi) {
    const int m = (lo + hi) >> 1;
    if (x0of(m) + 63 >= 0) hi = m; else lo = m + 1;
  }
  const int p_lo = lo;
  hi = nb;               // p_hi: the first p with x0 >= nrt
  while (lo < hi) {
    const int m = (lo + hi) >> 1;
    if (x0of(m) >= nrt) hi = m; else lo = m + 1;
  }
  const int p_hi = lo;
  // (slice, owner) pairs in ascending order, four at a time: the 16 loads of a group are in
  // flight together, then added owner by owner (the order of the sum does not change)
  constexpr int G = 4;
  const int no = p_hi - p_lo, nq = nh * no;
  for (int q0 = 0; q0 < nq; q0 += G) {
    f32x4 ld[G][4];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int q = q0 + u, j = q / no, p = p_lo + (q - j * no);
      const int x0 = x0of(p);
      const float* base = prow + ((int64_t)(i0 + j * hstep) * nb + p) * (int64_t)nrt * kHeadDim;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 4 * t + 1024 * k, x = x0 + (e >> 6);
        ld[u][k] = (q < nq && x >= 0 && x < nrt)
                       ? *(const f32x4*)(base + (int64_t)x * kHeadDim + (e & 63)) : f32x4{};
      }
    }
#pragma unroll
    for (int u = 0; u < G; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] += ld[u][k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = 4 * t + 1024 * k, row = row0 + (e >> 6), d = e & 63;
    if (row >= nrel) continue;
    f32x4 o = acc[k];
    if (head_last) {
      const int delta = row - off;
      o = f32x4{};
      if (delta > -L && delta < L && !shared) {
        const float dg = diag[(int64_t)h * (2 * L - 1) + delta + L - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = fmaf(v[(int64_t)h * kHeadDim + d + i], dg, acc[k][i]) * s;
      } else if (delta > -L && delta < L) {
        f32x4 vd = {};
        for (int hh = 0; hh < H; ++hh) {
          const float dg = diag[(int64_t)hh * (2 * L - 1) + delta + L - 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) vd[i] = fmaf(v[(int64_t)hh * kHeadDim + d + i], dg, vd[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (acc[k][i] + vd[i]) * s;
      }
    }
    *(f32x4*)(dr + ((int64_t)h * nrel + row) * kHeadDim + d) = o;
  }
}

// T-XL dv[h][d] = s sum_delta diag_h[delta] r_h[row(delta)][d]
template <typename T>
__global__ __launch_bounds__(1024) void agg_txl_dv_kernel(const float* __restrict__ diag,
                                                          const T* __restrict__ r, int64_t r_hs,
                                                          int L, int nrel, int off, float s,
                                                          float* __restrict__ dv) {
  // one workgroup per (head, 8 columns): thread t takes the offsets t, t + 1024, ..., reading 8
  // consecutive columns of each table row; then a fixed-order tree over the 1024 threads
  __shared__ float sh[8][1024];
  const int h = blockIdx.x >> 3, d0 = 8 * (blockIdx.x & 7);
  const int t = threadIdx.x;
  const int n = 2 * L - 1;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int x = t; x < n; x += 1024) {
    const int row = x - (L - 1) + off;
    if (row >= 0 && row < nrel) {
      float rv[8];
      load8(r + (int64_t)h * r_hs + (int64_t)row * kHeadDim + d0, rv);
      const float dg = diag[(int64_t)h * n + x];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(dg, rv[i], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sh[i][t] = acc[i];
  __syncthreads();
  for (int st = 512; st > 0; st >>= 1) {
    if (t < st) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sh[i][t] += sh[i][t + st];
    }
    __syncthreads();
  }
  if (t < 8) dv[(int64_t)h * kHeadDim + d0 + t] = sh[t][0] * s;
}

// T-XL du[h][d] = s sum_{b, block} part_kv[own][d]: one workgroup per head; thread t sums the
// owners of group t / 64 (64 consecutive owners each, in order) for column t % 64, and the four
// group sums are added in group order
__global__ __launch_bounds__(256) void agg_txl_du_kernel(const float* __restrict__ pkv, int B,
                                                         int H, int nb, float s,
                                                         float* __restrict__ du) {
  __shared__ float sh[4][kHeadDim];
  const int h = blockIdx.x, t = threadIdx.x, d = t & 63, g = t >> 6;
  const int nown = B * nb, per = (nown + 3) / 4;
  const int q0 = g * per, q1 = min(nown, q0 + per);
  float acc = 0.f;
#pragma unroll 8
  for (int q = q0; q < q1; ++q) {
    const int b = q / nb, p = q - b * nb;
    acc += pkv[(((int64_t)b * H + h) * nb + p) * kHeadDim + d];
  }
  sh[g][d] = acc;
  __syncthreads();
  if (t < kHeadDim) du[(int64_t)h * kHeadDim + t] = (((sh[0][t] + sh[1][t]) + sh[2][t]) + sh[3][t]) * s;
}

// ALiBi dm[h] = -sum over the (batch, query block) owners of head h of their sums of
// dS |i - j|, in ascending owner order.
__global__ void agg_alibi_kernel(const float* __restrict__ part, int B, int H, int nb,
                                 float* __restrict__ dm) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float acc = 0.f;
  for (int b = 0; b < B; ++b)
    for (int p = 0; p < nb; ++p) acc += part[((int64_t)b * H + h) * nb + p];
  dm[h] = -acc;
}

static inline int nblk(int64_t n, int t) { return (int)((n + t - 1) / t); }

hipError_t launch_agg_rows(const float* part, int64_t stride, int nown, int64_t nelem, float scale,
                           float* out, hipStream_t st) {
  if (nelem == 0) return hipSuccess;
  hipLaunchKernelGGL(agg_rows_kernel, dim3(nblk(nelem, 64)), dim3(256), 0, st, part, stride, 1,
                     nown, (int64_t)0, nelem, scale, out);
  return hipGetLastError();
}

hipError_t launch_agg_rows_by_head(const float* part, int64_t stride, int B, int H, int nb,
                                   int64_t nelem, float scale, float* out, hipStream_t st) {
  if (nelem == 0 || H == 0) return hipSuccess;
  hipLaunchKernelGGL(agg_rows_kernel, dim3(nblk(nelem, 64), H), dim3(256), 0, st, part, stride, B,
                     nb, (int64_t)H * nb, nelem, scale, out);
  return hipGetLastError();
}

hipError_t launch_agg_diag(const float* pdiag, int B, int H, int L, int nb, bool rev, int wl,
                           int wr, float* diag, hipStream_t st) {
  const int64_t nw = (int64_t)H * ((2 * L - 1 + 63) / 64);
  if (L < 1 || nw == 0) return hipSuccess;
  const bool compact = diag_width(L, wl, wr) != L + 256;
  const dim3 grid((unsigned)nw), blk(compact ? 1024 : 256);
  if (rev && compact)
    hipLaunchKernelGGL((agg_diag_kernel<true, true>), grid, blk, 0, st, pdiag, B, H, L, nb, wl, wr, diag);
  else if (rev)
    hipLaunchKernelGGL((agg_diag_kernel<true, false>), grid, blk, 0, st, pdiag, B, H, L, nb, wl, wr, diag);
  else if (compact)
    hipLaunchKernelGGL((agg_diag_kernel<false, true>), grid, blk, 0, st, pdiag, B, H, L, nb, wl, wr, diag);
  else
    hipLaunchKernelGGL((agg_diag_kernel<false, false>), grid, blk, 0, st, pdiag, B, H, L, nb, wl, wr, diag);
  return hipGetLastError();
}

hipError_t launch_agg_alibi(const float* part, int B, int H, int nb, float* dm, hipStream_t st) {
  hipLaunchKernelGGL(agg_alibi_kernel, dim3(nblk(H, 64)), dim3(64), 0, st, part, B, H, nb, dm);
  return hipGetLastError();
}

hipError_t launch_agg_txl_dr(const float* prow, const float* diag, const float* v, int H, int L,
                             int nb, int nrk, int wl, int wr, int nrel, int off, float s, int s0,
                             int ns, int nslices, bool first, bool last, bool shared, float* dr,
                             hipStream_t st) {
  const int nch = (nrel + 63) / 64;
  // the heads with a slice in the group [s0, s0 + ns): ns consecutive slices cover min(ns, H)
  // consecutive heads (mod H) from s0 mod H
  const int heads = shared ? 1 : std::min(ns, H);
  if (heads <= 0 || nch <= 0) return hipSuccess;
  hipLaunchKernelGGL(agg_txl_dr_kernel, dim3(heads * nch), dim3(256), 0, st, prow, diag,
                     v, H, L, nb, nrk, wl, wr, nrel, off, s, s0, ns, nslices, first ? 1 : 0, last ? 1 : 0,
                     shared ? 1 : 0, dr);
  return hipGetLastError();
}

hipError_t launch_agg_txl_uv(const float* pkv, const float* diag, const void* r, int64_t r_hs,
                             int B, int H, int L, int nb, int nrel, int off, float s, bool fp32,
                             float* du, float* dv, hipStream_t st) {
  if (fp32)
    hipLaunchKernelGGL((agg_txl_dv_kernel<float>), dim3(H * 8), dim3(1024), 0, st, diag,
                       (const float*)r, r_hs, L, nrel, off, s, dv);
  else
    hipLaunchKernelGGL((agg_txl_dv_kernel<uint16_t>), dim3(H * 8), dim3(1024), 0, st, diag,
                       (const uint16_t*)r, r_hs, L, nrel, off, s, dv);
  hipLaunchKernelGGL(agg_txl_du_kernel, dim3(H), dim3(256), 0, st, pkv, B, H, nb, s, du);
  return hipGetLastError();
}

}  // namespace relpos
