// Kernel argument blocks and launcher declarations shared by the host dispatcher and the
// kernel translation units.  Plain structs, passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace relpos {

enum { MECH_T5 = 0, MECH_SHAW = 1, MECH_TXL = 2, MECH_DEBERTA = 3 };
// ALiBi: a per-offset LUT like T5, with kernels of its own (its ramps replace the LUT on the
// tiles that lie on one side of the diagonal).
constexpr int MECH_ALIBI = 4;

constexpr int kHeadDim = 64;
constexpr int kMaxThresholds = 64;
constexpr int kMaxBuckets = 256;   // T5 buckets per head

// Per-offset dS partials of the query-side pass (T5, T-XL): one row of diag_width floats per
// wave of each 128-row block.  A full sweep keeps every offset: wave w of the block at A0 stores
// offset lam at lam - (A0 + 32 w - L - 64).  With a two-sided window the row keeps only the
// offsets of the wave's own sweep, counted from its last 64-row tile: the index is lowered by
// diag_xoff (at most wl + wr + 286 offsets; the compact form is used only when it is smaller).
__host__ __device__ inline int diag_width(int L, int wl, int wr) {
  const int64_t full = (int64_t)L + 256;
  if (wl < 0 || wr < 0) return (int)full;
  const int64_t w = ((int64_t)wl + wr + 286 + 63) / 64 * 64;
  return (int)(w < full ? w : full);
}
__host__ __device__ inline int diag_xoff(int L, int wl, int wr, int A0) {
  if (diag_width(L, wl, wr) == L + 256) return 0;
  int64_t bhi = (int64_t)A0 + 127 + wr;   // last streamed row of the sweep
  if (bhi > L - 1) bhi = L - 1;
  return L + 1 - (int)(bhi / 64 * 64);
}

// T5 bucket map: magnitude n >= max_exact lands in max_exact + #{e : n >= thr[e]}.
struct T5Map {
  int bidirectional;
  int half;        // buckets per direction (upper half offset when bidirectional)
  int max_exact;
  int nthr;        // log buckets - 1
  int thr[kMaxThresholds];
};

// Everything the attention kernels need to know about one call.
struct AttnShape {
  int B, H, L;
  int wl, wr;       // window; -1 = unbounded
  int mech;
  int span;         // Shaw / DeBERTa k
  int nrel;         // T-XL table rows
  int txl_off;      // T-XL row = delta + txl_off
  float scale;      // s
  int64_t rel_hs;   // elements between the relation tables of consecutive heads (0 = shared)
  int nbk;          // T5 buckets per head (else 0)
  // T5: every offset delta >= t5sat lands in bucket t5b_pos and every delta <= -t5sat in bucket
  // t5b_neg (the last bucket of each side); a huge t5sat for the other mechanisms
  int t5sat, t5b_pos, t5b_neg;
};

struct FwdArgs {
  AttnShape sh;
  const void* q;
  const void* k;
  const void* v;
  const void* rel_a;   // Shaw w, T-XL r, DeBERTa Kr
  const void* rel_b;   // DeBERTa Qr
  void* o;
  float* lse;
  const float* lut;    // T5: beta[bucket(delta)] / s per head, [H, 2L - 1]
  const float* uk;     // T-XL: u_h . k_j, [B, H, L]
  const float* vr;     // T-XL: v_h . r_h[row], [H, nrel]
  const float* rowc;   // Shaw / DeBERTa: per-query clipped-end products, [B, H, L, 2]
  const float* keyc;   // DeBERTa: per-key clipped-end p2c products, [B, H, L, 2]
  const int* bucket;   // T5: bucket of every offset, [2L - 1]
  const float* slopes; // ALiBi: m per head, [H]
};

struct BwdArgs {
  AttnShape sh;
  int bh0;             // first (batch, head) slice of this launch (b-major: b H + h)
  int nbh;             // slices in this launch (0 = all B H)
  int fold;            // general passes of Shaw / DeBERTa: batch entries per partial slot (>= 1),
  int fold_slices;     // ... or, with a table shared by every head, (batch, head) slices per slot
  int sub;             // run as `fold` launches, this one taking entry `sub` of each group
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* dsum;   // D_i = dO_i . O_i, [B, H, L]
  const void* rel_a;
  const void* rel_b;
  const float* lut;
  const float* uk;
  const float* vr;
  const float* rowc;
  const float* keyc;
  const int* bucket;
  const float* bias_a; // T-XL u
  const float* bias_b; // T-XL v
  void* dq;
  void* dk;
  void* dv;
  float* part_q;       // query-side partials (dQ pass)
  float* part_k;       // key-side partials (dK/dV pass)
  float* part_qv;      // query-side per-owner small vectors (T5 bucket sums, T-XL diagonal
                       // sums, ALiBi slope sums)
  float* part_kv;      // key-side per-owner small vectors (T-XL du)
  int64_t part_q_stride;  // floats per owner
  int64_t part_k_stride;
  float* xpart;        // split passes: fp32 dX from the clipped steps, [B, H, L, 64]
  float* vpart;        // split key-side pass: fp32 dV from the clipped steps
  float* cab;          // split passes: end-row sums of dS per lane row, [B, H, L, 2]
};

// ----------------------------------------------------------------------------- launchers
// Each returns a hipError_t from hipGetLastError() after enqueueing on `stream`.
hipError_t launch_fwd(const FwdArgs& a, bool fp32, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, bool fp32, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, bool fp32, hipStream_t stream);

// out[n * ne + e] = x_n . y_e(h(n)) for rows x_n of length 64.  Row n belongs to head
// h(n) = (n / rows_per_head) % H; x_n = x + 64 n when x_head_stride < 0 (dense rows), else
// x + h(n) x_head_stride + 64 (n % rows_per_head); y_e(h) = y + h y_head_stride + 64 y_row[e].
struct RowDotArgs {
  const void* x;
  int64_t nrows;
  int64_t rows_per_head;
  int H;
  const void* y;
  int64_t y_head_stride;
  int y_row0, y_row1;
  int ne;
  float* out;
  int64_t x_head_stride;
};
hipError_t launch_rowdot(const RowDotArgs& a, bool x_fp32, bool y_fp32, hipStream_t stream);

// ALiBi LUT: lut[h][delta + L - 1] = -m_h |delta| * inv_scale
hipError_t launch_alibi_lut(const float* slopes, int H, int L, float inv_scale, float* lut,
                            hipStream_t stream);
hipError_t launch_t5_lut(const float* beta, int H, int L, int nb, float inv_scale, const T5Map& m,
                         float* lut, hipStream_t stream);
hipError_t launch_index_map(int mech, int L, int span, int nrel, int txl_off, const T5Map& m,
                            int32_t* out_a, int32_t* out_b, hipStream_t stream);
// second-pass aggregation of the backward's offset-sharded partials: out = scale * the sum of
// the nown partials (slots 0 .. nown - 1, each `stride` floats apart), in a fixed order
hipError_t launch_agg_rows(const float* part, int64_t stride, int nown, int64_t nelem, float scale,
                           float* out, hipStream_t st);
// the same per head: owners are slots (b H + h) nb + p; out[h nelem + e] sums head h's owners
// (b, p) in ascending order
hipError_t launch_agg_rows_by_head(const float* part, int64_t stride, int B, int H, int nb,
                                   int64_t nelem, float scale, float* out, hipStream_t st);
hipError_t launch_agg_diag(const float* pdiag, int B, int H, int L, int nb, bool rev, int wl,
                           int wr, float* diag, hipStream_t st);
// ALiBi dm[h] = -sum over the owners (b, query block) of head h of part[owner] (fixed order)
hipError_t launch_agg_alibi(const float* part, int B, int H, int nb, float* dm, hipStream_t st);
// T-XL dr from the key-side r partials of the slice group [s0, s0 + ns) of nslices slices
// (partial slot of slice s0 + i, key block p: i nb + p), summed in ascending (slice, block)
// order.  Groups are added in order, each launched for the heads with a slice in it: a head's
// first group overwrites its dr, later ones add to it; its dr holds raw sums until its last
// group, which adds v . diag and scales by s.  With `shared` one table serves every head:
// dr [nrel, 64] sums the slices of every head, `first` / `last` mark the first and last group,
// and the diagonal term is sum_h v_h . diag_h.
hipError_t launch_agg_txl_dr(const float* prow, const float* diag, const float* v, int H, int L,
                             int nb, int nrk, int wl, int wr, int nrel, int off, float s, int s0,
                             int ns, int nslices, bool first, bool last, bool shared, float* dr,
                             hipStream_t st);
// T-XL dv (v . r diagonal term; head h reads r + h r_hs) and du (from the key-side per-owner
// sums of dS^T k)
hipError_t launch_agg_txl_uv(const float* pkv, const float* diag, const void* r, int64_t r_hs,
                             int B, int H, int L, int nb, int nrel, int off, float s, bool fp32,
                             float* du, float* dv, hipStream_t st);

// Relation-table projections: rel [H, N, d] = X [N, F] . W [F, H d] (dtype of X and W; rel
// written in that dtype), and the backward dX = dY . W^T [N, F], dW = X^T . dY [F, H d] (fp32)
// with dY(n, h d + c) = drel[h][n][c].  dW sums `kslices` fp32 slices of the n range held in
// `partials` ([kslices, F, H d]; unused when kslices == 1).  Either of dX / dW may be null.
// F, d multiples of 8; pointers 16-byte aligned.
hipError_t launch_project_fwd(const void* X, const void* W, void* rel, int N, int F, int H, int d,
                              bool fp32, hipStream_t st);
hipError_t launch_project_bwd(const void* X, const void* W, const float* drel, float* dX, float* dW,
                              float* partials, int kslices, int N, int F, int H, int d, bool fp32,
                              hipStream_t st);

// D_n = dO_n . O_n over rows of length 64
hipError_t launch_dsum(const void* o, const void* dout, int64_t nrows, bool fp32, float* dsum,
                       hipStream_t stream);

}  // namespace relpos
