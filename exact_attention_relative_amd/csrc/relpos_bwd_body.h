#pragma once
// Backward kernels.  One template, instantiated twice per mechanism:
//   DIR 0: lane side = queries (128 per workgroup), keys streamed: dQ and the query-side table
//          gradients (Shaw w, T-XL r and its diagonal sums, DeBERTa Kr, T5 bucket sums).
//   DIR 1: lane side = keys, queries streamed: dK, dV and the key-side table gradient
//          (DeBERTa Qr), plus the T-XL u gradient.
// Both recompute S and P = exp(S - LSE) per tile exactly as the forward does and form
// dS = P (dP - D) in fp32.  Relation products are reused in both directions (abstract,
// item 2).  Table gradients follow offset-based gradient sharding (abstract, item 3; zicq.com
// explainer, section on offset-based gradient sharding): each workgroup accumulates, per
// offset, the sum over its own rows in registers and writes every offset of its partial
// exactly once; a second pass (relpos_agg.hip) merges the partials in a fixed order, so results
// are bitwise reproducible.  The general passes of Shaw and DeBERTa may run the batch entries of
// a head as consecutive launches into one partial: the first stores it, each later launch adds
// to every element once (an atomic add; one per element and launch, launches in stream order,
// so each element's sum keeps one order).  T5 sums dS per bucket in LDS instead.
//
// Relation gradients of a table applied on one side (the row side: lane rows X times the table
// row of offset lam = a - b) are split over the two passes so that each fits two workgroups per
// CU.  The pass where the table is on the row side adds dX_rel = sum_b dS[a][b] T[row(lam)]
// with the skewed operand read straight from the wave's fp32 dS buffer; the pass where it is
// on the column side (the X rows are now the streamed rows) runs the table GEMM over its
// streamed tile,
//   dT_window[t] += sum_y E2[t][y] Y[y],   E2[t][y] = dS[y][x], t = y - x + 127,
// with E2 in the space of the column-side skew buffer.  The window slides by 64 offsets per
// step, so a wave's three 32-offset accumulators shift each step and the one that leaves the
// window is final: it is written out.  T-XL (full span, every tile general) runs this over every
// step.  Shaw and DeBERTa (clipped offsets) run each direction in two parts: a light pass over
// the steps whose workgroup tile is clipped throughout (every element reads an end row, so the
// relation term is a per-row constant) and a general pass over the rest; the table's interior
// rows come from the column-side general pass, its two end rows (sums over the clipped
// elements) from the row-side passes.
#include "relpos_tile.h"

namespace relpos {

constexpr int ESTRT = 200;    // bf16 E2T row stride (elements): 192 window offsets + pad

// PART 0: the whole sweep.  PART 1 (light): only the steps whose workgroup tile is clipped
// (every offset beyond the span), without any relation-product machinery, writing fp32 partial
// dX / dV and the end-row sums.  PART 2: only the contiguous range of general steps, merging
// the light pass's partials into the final outputs.
template <int MECH, int DIR, int PART>
struct BV {
  static constexpr bool LUTP = MECH == MECH_T5 || MECH == MECH_ALIBI;   // per-offset bias LUT
  static constexpr bool HAS_ROW = DIR == 0 ? !LUTP : MECH == MECH_DEBERTA;
  static constexpr bool HAS_COL = DIR == 0 ? MECH == MECH_DEBERTA : !LUTP;
  static constexpr bool LIGHT = PART == 1;
  static constexpr bool FAT = PART == 2;
  static constexpr bool ROW = HAS_ROW && !LIGHT;
  static constexpr bool COL = HAS_COL && !LIGHT;
  static constexpr bool TXL = MECH == MECH_TXL;
  static constexpr bool CLIP = MECH == MECH_SHAW || MECH == MECH_DEBERTA;
  static constexpr bool DIAG = DIR == 0 && (MECH == MECH_T5 || MECH == MECH_TXL);
  // T5: the per-offset sums go straight into per-bucket sums of the workgroup
  static constexpr bool T5BIN = DIAG && MECH == MECH_T5;
  // General pass of Shaw / DeBERTa: the row-side dX_rel from the wave's dS buffer and the
  // column-side table gradient over the streamed rows (no workgroup band buffer, so two
  // workgroups fit per CU); a table's interior rows come from the pass where it is the column
  // side, its end rows from the pass where it is the row side
  static constexpr bool DFAT = CLIP && PART == 2;
  static constexpr bool TQ = TXL && DIR == 0;         // T-XL query side (circular row window)
  static constexpr bool TK = TXL && DIR == 1;         // T-XL key side (circular column window)
  static constexpr bool GSREL = TQ || (DFAT && HAS_ROW);   // dX_rel from the wave's dS buffer
  static constexpr bool TG1 = TK || (DFAT && HAS_COL);     // table GEMM over the streamed rows
  static constexpr bool WINB = ROW || COL;
  static constexpr bool GSB = ROW || COL || DIAG;

  // row-side table row of lane offset lam = a - b
  __device__ static int row_of(int lam, int span, int nrel, int off) {
    if (DIR == 0) return row_side_row(MECH, lam, span, nrel, off);
    return clampi(lam + span, 0, 2 * span - 1);   // DeBERTa p2c: lam = j - i
  }
  // column-side table row of other offset mu = b - a
  __device__ static int col_of(int mu, int span, int nrel, int off) {
    if (DIR == 0) return clampi(mu + span, 0, 2 * span - 1);   // DeBERTa p2c: mu = j - i
    return row_side_row(MECH, mu, span, nrel, off);             // mu = i - j
  }
  // offsets <= TA share end row A, >= TB share end row B (Shaw / DeBERTa only)
  __device__ static int TA(int span) { return -span; }
  __device__ static int TB(int span) { return MECH == MECH_SHAW ? span : span - 1; }
  __device__ static int rowA(int span) { return MECH == MECH_SHAW ? 2 * span : 0; }
  __device__ static int rowB(int span) { return MECH == MECH_SHAW ? 0 : 2 * span - 1; }
};

// ----------------------------------------------------------------------------- kernel
// T is the element type of the inputs (uint16_t = bf16 bits, or float); fp32 operands enter the
// matrix cores as NP = 2 bf16 planes (hi, lo), with every LDS tile holding both planes.
// FIRSTK: 1 or 0 fixes at compile time whether this launch stores its partials (the first of
// a folded pass) or adds to them; -1 reads it from the arguments.
template <typename T, int MECH, int DIR, int PART, int FIRSTK = -1>
__device__ __forceinline__ void bwd_body(const BwdArgs& a) {
  using V = BV<MECH, DIR, PART>;
  constexpr int NP = Elem<T>::NP;
  __shared__ __attribute__((aligned(16))) uint16_t ys[NP * BOTH * TSTR];    // K (dir 0) / Q (dir 1)
  __shared__ __attribute__((aligned(16))) uint16_t y2s[NP * BOTH * TSTR];   // V (dir 0) / dO (dir 1)
  __shared__ __attribute__((aligned(16))) uint16_t win[V::WINB ? NP * WIN * TSTR : 8];
  // the skewed reads of the dX_rel operand reach up to 32 floats beyond a wave's buffer
  constexpr int GSG = V::GSREL ? 32 : 0;
  // the buffer also holds the E2T band (NP planes of BOTH x ESTRT bf16) when there is a table
  // GEMM, and the end-row staging (2 BLANE sums and BLANE lane rows) of the general passes
  constexpr int GS_SKEW = V::GSB ? NWAVE * WROWS * GS2 + 2 * GSG : 4;
  constexpr int GS_E2T = V::TG1 ? NP * BOTH * ESTRT / 2 + GSG : 0;
  constexpr int GS_END = (V::DFAT && V::ROW) ? 2 * BLANE + NP * BLANE * TSTR / 2 + GSG : 0;
  constexpr int GS_ALL = GS_SKEW > GS_E2T ? (GS_SKEW > GS_END ? GS_SKEW : GS_END)
                                          : (GS_E2T > GS_END ? GS_E2T : GS_END);
  __shared__ __attribute__((aligned(16))) float gsb_raw[GS_ALL];
  __shared__ __attribute__((aligned(16))) float vec_s[V::LUTP ? WIN : 4];  // bias LUT slice
  // T-XL u.k / clipped end-row constants / ALiBi ramps +m y / s and -m y / s
  constexpr int NOVEC = (MECH == MECH_TXL && DIR == 0)
                            ? BOTH
                            : ((V::CLIP && V::HAS_COL && !V::DFAT) || MECH == MECH_ALIBI ? 2 * BOTH : 4);
  __shared__ float red_s[MECH == MECH_ALIBI ? NWAVE : 1];   // ALiBi: per-wave slope-gradient sums
  __shared__ float bins_s[V::T5BIN ? NWAVE * kMaxBuckets : 1];   // T5: per-wave bucket sums of dS
  __shared__ __attribute__((aligned(16))) float ovec_s[NOVEC];   // per-other-row constants
  // key side: -LSE / s and -D of the streamed queries, the starts of the score and dP
  // accumulators (y units; -inf for rows past L or with no allowed key; see lsd_vals)
  __shared__ __attribute__((aligned(16))) float lsd_s[DIR == 1 ? 2 * BOTH : 4];
  // Key side: the score and dP accumulators start from those values (one fma and one multiply per
  // element instead of two of each), except in the T-XL pass, whose registers are the limit
  constexpr bool KINIT = DIR == 1 && !V::TK;
  // key-side ALiBi: the ramps above plus -LSE / s, per step
  __shared__ __attribute__((aligned(16))) float ainit_s[MECH == MECH_ALIBI && DIR == 1 ? 2 * BOTH : 4];
  float* const gsb = gsb_raw + GSG;

  const AttnShape sh = a.sh;
  const int L = sh.L;
  const int nb = (L + BLANE - 1) / BLANE;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int blk = bid % nb;
  int bh = a.bh0 + bid / nb;
  // folded pass (general passes of Shaw and DeBERTa, T-XL key side): launch `sub` of `fold`
  // runs batch entry bg fold + sub of head h in workgroup group g = bg H + h, or, for a table
  // every head shares (fold_slices), slice g fold + sub; the first launch stores the group's
  // partial slot, the later ones add to it
  constexpr bool FOLDS = V::DFAT || V::TK;
  const bool first = FIRSTK >= 0 ? FIRSTK == 1 : (!FOLDS || a.sub == 0);
  if constexpr (FOLDS) {
    if (a.fold > 1) {
      const int g = bid / nb;
      if (a.fold_slices) {
        bh = g * a.fold + a.sub;
        if (bh >= sh.B * sh.H) return;
      } else {
        const int bb = (g / sh.H) * a.fold + a.sub;
        if (bb >= sh.B) return;
        bh = bb * sh.H + g % sh.H;
      }
    }
  }
  if (sh.wr == 0) blk = (DIR == 0) ? nb - 1 - blk : blk;   // causal: longest first
  const int h = bh % sh.H;
  const int A0 = blk * BLANE;
  const int tid = threadIdx.x;
  const int w = wave_index(), lane = tid & 63, l32 = lane & 31, kh = lane >> 5;
  const int aw0 = A0 + WROWS * w;
  const int my_a = aw0 + l32;
  const int span = sh.span, nrel = sh.nrel, toff = sh.txl_off;
  const float s = sh.scale, c = s * kLog2e;
  const int64_t bh_off = (int64_t)bh * L * kHeadDim;
  const int64_t owner = (int64_t)a.bh0 * nb + bid;   // partial slot of this workgroup

  const T* xg = (const T*)(DIR == 0 ? a.q : a.k) + bh_off;
  const T* x2g = (const T*)(DIR == 0 ? a.dout : a.v) + bh_off;
  const T* yg = (const T*)(DIR == 0 ? a.k : a.q) + bh_off;
  const T* y2g = (const T*)(DIR == 0 ? a.v : a.dout) + bh_off;
  // this head's tables (rel_hs = 0: one table shared by every head)
  const T* trow = (const T*)(DIR == 0 ? a.rel_a : a.rel_b);   // row-side table
  const T* tcol = (const T*)(DIR == 0 ? a.rel_b : a.rel_a);   // column-side table
  if (trow) trow += h * sh.rel_hs;
  if (tcol) tcol += h * sh.rel_hs;
  const float* rc_g = DIR == 0 ? a.rowc : a.keyc;   // lane rows . row table ends (A, B)
  const float* oc_g = DIR == 0 ? a.keyc : a.rowc;   // other rows . column table ends (A, B)

  // ---- lane-side registers ----
  Op<NP> xop[4], x2op[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    if (my_a < L) {
      xop[cc] = op_from_global<T>(xg + (int64_t)my_a * kHeadDim + 16 * cc + 8 * kh);
      x2op[cc] = op_from_global<T>(x2g + (int64_t)my_a * kHeadDim + 16 * cc + 8 * kh);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      xop[cc] = op_from_f32<NP>(z);
      x2op[cc] = xop[cc];
    }
  }
  float lse2 = __builtin_inff(), dsum_l = 0.f;   // dir 0: per lane
  if (DIR == 0 && my_a < L) {
    lse2 = a.lse[(int64_t)bh * L + my_a] * kLog2e;
    dsum_l = a.dsum[(int64_t)bh * L + my_a];
    if (!(lse2 > kNegInf)) lse2 = __builtin_inff();   // empty row: P = 0
  }
  float rcA = 0.f, rcB = 0.f;
  if constexpr (V::CLIP && V::HAS_ROW && !V::DFAT) {
    if (my_a < L) {
      rcA = rc_g[((int64_t)bh * L + my_a) * 2 + 0];
      rcB = rc_g[((int64_t)bh * L + my_a) * 2 + 1];
    }
  }
  float ukl = 0.f;   // dir 1 T-XL: u . k of this lane's key
  if constexpr (MECH == MECH_TXL && DIR == 1) {
    if (my_a < L) ukl = a.uk[(int64_t)bh * L + my_a];
  }

  // ---- sweep range over the other side ----
  int b_lo = 0, b_hi = L - 1;
  if (DIR == 0) {
    if (sh.wl >= 0) b_lo = max(0, A0 - sh.wl);
    if (sh.wr >= 0) b_hi = min(L - 1, A0 + BLANE - 1 + sh.wr);
  } else {
    if (sh.wr >= 0) b_lo = max(0, A0 - sh.wr);
    if (sh.wl >= 0) b_hi = min(L - 1, A0 + BLANE - 1 + sh.wl);
  }
  const int bt_all = (b_lo / BOTH) * BOTH;
  const int nsteps_all = (b_hi >= b_lo) ? (b_hi - bt_all) / BOTH + 1 : 0;
  // workgroup tile of step base b0 needs relation products (some offset not clipped)
  auto wg_gen = [&](int b0) {
    if constexpr (V::CLIP) {
      const int ta = V::TA(span), tb = V::TB(span);
      const int wlo = A0 - b0 - 63, whi = A0 - b0 + 127;
      const bool gr = V::HAS_ROW && !(whi <= ta || wlo >= tb);
      const bool gc = V::HAS_COL && !(-wlo <= ta || -whi >= tb);
      return gr || gc;
    }
    return true;
  };
  // the general steps form one contiguous range (the window slides monotonically)
  int g_first = nsteps_all, g_last = -1;
  if constexpr (PART != 0) {
    for (int s2 = 0; s2 < nsteps_all; ++s2)
      if (wg_gen(bt_all + s2 * BOTH)) { g_first = min(g_first, s2); g_last = s2; }
  }
  const int bt0 = V::FAT ? bt_all + g_first * BOTH : bt_all;
  const int nsteps = V::FAT ? (g_last >= g_first ? g_last - g_first + 1 : 0) : nsteps_all;
  const int bt_last = bt0 + (nsteps - 1) * BOTH;

  // ---- partial layouts ----
  // lane offsets lam of this workgroup lie in [lam_base, lam_base + L + 256)
  const int lam_base = A0 - L - 64;
  float* prow = nullptr;     // row-side table partial
  int prow_rows = 0;
  if constexpr (V::DFAT) {
    prow_rows = (MECH == MECH_SHAW) ? 2 * span + 1 : 2 * span;
    prow = (DIR == 0 ? a.part_q : a.part_k) + owner * (DIR == 0 ? a.part_q_stride : a.part_k_stride);
  }
  // DeBERTa general pass: column-side table partial (its interior rows; the end rows are the
  // other direction's row-side end rows)
  float* pcol = nullptr;
  if constexpr (V::DFAT)
    pcol = (DIR == 0 ? a.part_k : a.part_q) + owner * (DIR == 0 ? a.part_k_stride : a.part_q_stride);
  // T-XL r partial of the key-side pass: row b0 + 65 + t holds window row t of step base b0
  // (offset delta = b0 - A0 - 127 + t), i.e. row delta + A0 + 192
  // With a two-sided window the partial keeps only the rows of this sweep, from row bt0 + 65.
  float* ptg = nullptr;
  const int nrk = (int)(a.part_q_stride / kHeadDim);
  const int rb = (sh.wl >= 0 && sh.wr >= 0) ? bt0 + 65 : 0;
  // (slots of the r partial count from the launch's first slice)
  if constexpr (V::TK) ptg = a.part_q + (int64_t)bid * a.part_q_stride - (int64_t)rb * kHeadDim;
  // T-XL per-offset dS sums: one partial row of ndg floats per wave (lane offset lam at index
  // lam - (lam_base + 32 w) - dxo), in the owner's slot of NWAVE rows
  const int ndg = diag_width(L, sh.wl, sh.wr), dxo = diag_xoff(L, sh.wl, sh.wr, A0);
  float* pdiag = nullptr;
  if constexpr (V::DIAG && !V::T5BIN) pdiag = a.part_qv + owner * (int64_t)(NWAVE * ndg);
  // T5: each wave sums dS per bucket in its own LDS row; the workgroup's sums (nbk floats)
  // go to the owner's slot at the end
  float* const binw = bins_s + (V::T5BIN ? w * kMaxBuckets : 0);
  if constexpr (V::T5BIN) {
    for (int e = tid; e < NWAVE * kMaxBuckets; e += 256) bins_s[e] = 0.f;   // (first barrier below)
  }

  // ---- zero what the sweep will not write ----
  if (V::DFAT && V::HAS_COL && first) {
    // column offsets mu = b - a of every window row of every step are flushed (interior ones)
    // (table row of mu: Shaw k - mu, DeBERTa mu + k; the end rows, 0 and the last, come from
    // the row-side sums, so only interior rows outside the flushed range are cleared here)
    const int mlo = bt0 - A0 - (BLANE - 1), mhi = bt_last - A0 + BOTH;
    const int rlast = prow_rows - 2;   // last interior row
    int wl = rlast + 1, wh = rlast;    // flushed interior rows [wl, wh]
    if (nsteps > 0) {
      const int r0 = (MECH == MECH_SHAW) ? span - mhi : mlo + span;
      const int r1 = (MECH == MECH_SHAW) ? span - mlo : mhi + span;
      wl = clampi(r0, 1, rlast + 1);
      wh = clampi(r1, wl - 1, rlast);
    }
    for (int64_t e = kHeadDim + tid; e < (int64_t)wl * kHeadDim; e += 256) pcol[e] = 0.f;
    for (int64_t e = (int64_t)(wh + 1) * kHeadDim + tid; e < (int64_t)(rlast + 1) * kHeadDim; e += 256)
      pcol[e] = 0.f;
  }
  if (V::TK && first) {
    // the slot holds rows [rb, rb + nrk); the sweep writes [bt0 + 65, bt_last + 256], so only
    // the rows below and above that range are cleared here
    const int r_end = rb + nrk;
    const int w_lo = nsteps > 0 ? clampi(bt0 + 65, rb, r_end) : r_end;
    const int w_hi = nsteps > 0 ? clampi(bt_last + 257, w_lo, r_end) : r_end;
    float* zb = ptg + (int64_t)rb * kHeadDim;
    for (int64_t e = tid; e < (int64_t)(w_lo - rb) * kHeadDim; e += 256) zb[e] = 0.f;
    for (int64_t e = (int64_t)(w_hi - rb) * kHeadDim + tid; e < (int64_t)nrk * kHeadDim; e += 256) zb[e] = 0.f;
  }
  if constexpr (V::DIAG && !V::T5BIN) {
    // wave ww writes the offsets [A0 + 32 ww - bt_last - 63, A0 + 32 ww - bt0 + 32], i.e.
    // entries [klo, khi] of its row (entry k: lam = lam_base + 32 ww + dxo + k), the same range
    // in every wave's row; the rest of each row is cleared here
    int klo = ndg, khi = ndg - 1;
    if (nsteps > 0) {
      klo = clampi(A0 - bt_last - 63 - lam_base - dxo, 0, ndg);
      khi = clampi(A0 - bt0 + 32 - lam_base - dxo, klo - 1, ndg - 1);
    }
#pragma unroll
    for (int ww = 0; ww < NWAVE; ++ww) {
      float* prw = pdiag + ww * ndg;
      for (int k = tid; k < klo; k += 256) prw[k] = 0.f;
      for (int k = khi + 1 + tid; k < ndg; k += 256) prw[k] = 0.f;
    }
  }

  // ---- accumulators ----
  f32x16 gacc[2] = {f32x16{}, f32x16{}};    // dX (content + relation), dir 1: dK
  f32x16 vacc[2] = {f32x16{}, f32x16{}};    // dir 1: dV
  f32x16 racc[3] = {f32x16{}, f32x16{}, f32x16{}};   // table window accumulators
  float cA = 0.f, cB = 0.f;                  // clipped-end sums of dS (lane row)
  float colsum = 0.f;                        // dir 1 T-XL: sum_i dS_ij
  float dcarry = 0.f;                        // diagonal t = lane carried into the next step
  // T5: single-bucket wave tiles add to this lane's running sum while the bucket stays the
  // same (it changes a few times along a row of tiles); the lanes are summed and the bucket
  // updated only when it changes and after the last step, not once per step
  float t5acc = 0.f;
  int t5cur = -1;
  auto t5_flush = [&]() {
    if (t5cur >= 0) {
      float tot = t5acc + xhalf(t5acc);
      for (int m = 1; m < 32; m <<= 1) tot += __shfl_xor(tot, m);
      if (lane == 0) binw[t5cur] += tot;
    }
    t5acc = 0.f;
  };
  const int gdb = w & 1, gp = w >> 1;        // GEMM tiles of this wave: d-block, t-block parity
  // T-XL key side: the window block that leaves with a step is written to the r partial in
  // the next step, after that step's staging reads are issued: the vector-memory counter drains
  // in issue order, so reads issued after the partial's stores and atomics would wait for them
  // too.  (bf16; the fp32 pass writes it at once.)
  constexpr bool TK_DEFER = V::TK && NP == 1;
  f32x16 rflush = {};
  // (addressed from the slot's base rebuilt in scalar registers plus a 32-bit lane offset: a
  // per-lane 64-bit address would be spilled, and its reload waits for every read in flight)
  auto flush_r = [&](const f32x16& acc, int b0x) {
    typedef __attribute__((address_space(1))) float gfloat;
    gchar* base = scalar_ptr(ptg);
    const uint32_t off =
        4u * (uint32_t)((b0x + 65 + 32 * gp + 4 * kh) * kHeadDim + 32 * gdb + l32);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      gfloat* f = (gfloat*)(base + off + 4u * (uint32_t)((8 * (r >> 2) + (r & 3)) * kHeadDim));
      if (first) *f = acc[r];
      else __builtin_amdgcn_global_atomic_fadd_f32(f, acc[r]);
    }
  };

  // Store one window accumulator block to the column-side table partial: register r holds
  // offset mu0 + 8 (r / 4) + r % 4 (mu = b - a), column 32 gdb + l32.  Only interior offsets are
  // stored (clipped ones belong to the end rows); when the whole block is interior its 16 rows
  // are consecutive table rows (ascending for DeBERTa, row mu + k; descending for Shaw, k - mu),
  // stored from one base without per-element tests.
  // (a folded pass's later batch entries add to what the first stored)
  auto flush_col = [&](const f32x16& acc, int mu0) {
    const int d = 32 * gdb + l32;
    constexpr int rstep = (MECH == MECH_SHAW) ? -1 : 1;
    if (mu0 > V::TA(span) && mu0 + 27 < V::TB(span)) {
      float* fb = pcol + (uint32_t)(V::col_of(mu0, span, nrel, toff) * kHeadDim + d);
      if (first) {
#pragma unroll
        for (int r = 0; r < 16; ++r) fb[rstep * (8 * (r >> 2) + (r & 3)) * kHeadDim] = acc[r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) unsafeAtomicAdd(fb + rstep * (8 * (r >> 2) + (r & 3)) * kHeadDim, acc[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mu = mu0 + 8 * (r >> 2) + (r & 3);
        if (mu > V::TA(span) && mu < V::TB(span)) {
          float* f = pcol + (uint32_t)(V::col_of(mu, span, nrel, toff) * kHeadDim + d);
          if (first) *f = acc[r]; else unsafeAtomicAdd(f, acc[r]);
        }
      }
    }
  };
  float* gs = gsb + (V::GSB ? w * WROWS * GS2 : 0);

  // the next step's streamed tiles are read into registers while the current step computes
  auto step_base = [&](int st) { return bt0 + st * BOTH; };
  auto step_skipped = [&](int st) { return V::LIGHT && st >= g_first && st <= g_last; };
  // ALiBi: on a wave tile on one side of the diagonal, -m |i - j| / s = (lane-row term) +
  // (streamed-row term), the latter a ramp over the 64 streamed rows: the ramp starts the score
  // accumulators and the lane-row term is the lane constant, so those tiles add nothing per
  // element; straddling tiles read the per-offset LUT.  The query-side pass also accumulates
  // dm = -sum dS |i - j| per lane (the slope gradient), without per-offset sums.
  float am = 0.f, amacc = 0.f;
  if constexpr (MECH == MECH_ALIBI) {
    am = a.bias_a[h] / s;
    if (tid < BOTH) {
      ovec_s[tid] = am * (float)tid;
      ovec_s[BOTH + tid] = -am * (float)tid;
    }
  }
  // per-row values of the streamed rows (end-row constants of the light key-side passes, LSE
  // and D of the streamed queries), read one processed step ahead
  f32x2 pov = {0.f, 0.f};
  float pnl = 0.f, pdd = 0.f;
  const float inv_s = 1.f / s;
  auto colfn_at = [&](int b0x) {   // column window row x <-> mu = b - a = (b0 - A0 - 127) + x
    return [=](int x) { return V::col_of((b0x - A0 - (BLANE - 1)) + x, span, nrel, toff); };
  };
  auto rowfn_at = [&](int b0x) {   // row window row x <-> lam = A0 - b0 - 63 + x
    return [=](int x) { return V::row_of(A0 - b0x - 63 + x, span, nrel, toff); };
  };
  auto ov_load = [&](int b0x) {   // end A, end B values of streamed row b0x + tid (column side)
    if (tid < BOTH) {
      const int yy = b0x + tid;
      pov = (yy < L) ? *(const f32x2*)(oc_g + ((int64_t)bh * L + yy) * 2) : f32x2{0.f, 0.f};
    }
  };
  // key side: -LSE / s and -D of streamed query b0x + tid (the accumulator starts); the T-XL
  // pass keeps LSE log2 e (+inf for rows past L or with no allowed key) and D, applied per element
  auto lsd_vals = [&](int b0x, float& nl, float& nd) {
    const int yy = b0x + tid;
    if constexpr (KINIT) {
      nl = kNegInf;
      nd = 0.f;
      if (yy < L) {
        const float lse = a.lse[(int64_t)bh * L + yy];
        if (lse > kNegInf) nl = -lse * inv_s;
        nd = -a.dsum[(int64_t)bh * L + yy];
      }
    } else {
      nl = __builtin_inff();
      nd = 0.f;
      if (yy < L) {
        nl = a.lse[(int64_t)bh * L + yy] * kLog2e;
        if (!(nl > kNegInf)) nl = __builtin_inff();
        nd = a.dsum[(int64_t)bh * L + yy];
      }
    }
  };
  auto lsd_load = [&](int b0x) {
    if (tid < BOTH) lsd_vals(b0x, pnl, pdd);
  };
  float plut = 0.f;   // T5 / ALiBi: this thread's LUT entry of the next step's window
  auto lut_load = [&](int b0x) {
    if (tid < WIN) {
      const int lam = (A0 - b0x) - 63 + tid;
      const int d = DIR == 0 ? lam : -lam;
      plut = (d > -L && d < L) ? a.lut[(int64_t)h * (2 * L - 1) + d + L - 1] : 0.f;
    }
  };
  // the next processed step's per-row values are read while the current step computes (not in
  // the T-XL key-side pass, whose registers are the limit: it reads them with the step's own
  // batch of reads)
  constexpr bool PF_LSD = DIR == 1 && !V::TK;
  constexpr bool PF_OV = V::CLIP && V::HAS_COL && !V::DFAT;
  auto scalars_load = [&](int b0x) {
    if constexpr (PF_LSD) lsd_load(b0x);
    if constexpr (PF_OV) ov_load(b0x);
    if constexpr (V::LUTP) lut_load(b0x);
  };
  constexpr bool ANY_PF = PF_LSD || PF_OV || V::LUTP;
  int next = 0;
  while (next < nsteps && step_skipped(next)) ++next;
  if constexpr (ANY_PF) {
    if (next < nsteps) scalars_load(step_base(next));
  }
  TilePrefetch<T> py, py2;
  TilePrefetch<T> pwn;   // query-side T-XL: the next step's 64 new window rows
  float pvr = 0.f;       // and their v.r values (threads 0..63)
  float puk = 0.f;       // query-side T-XL: u.k of the next step's keys (threads 0..63)
  if constexpr (V::TQ) {
    if (tid < BOTH && nsteps > 0) puk = (bt0 + tid < L) ? a.uk[(int64_t)bh * L + bt0 + tid] : 0.f;
  }
  if (!V::TG1 && next < nsteps) {
    py.load(yg, step_base(next), L);
    py2.load(y2g, step_base(next), L);
  }

  for (int step = 0; step < nsteps; ++step) {
    const int b0 = bt0 + step * BOTH;
    // query-side T-XL: the row window slides by 64 offsets per step and is kept circular,
    // window row x of step s at physical row (x - 64 s) mod 192
    // key-side T-XL: the column window slides up by 64 per step, row x at (x + 64 s) mod 192
    const int xrot = V::TQ ? ((3 - step % 3) % 3) * BOTH : V::TK ? (step % 3) * BOTH : 0;
    if constexpr (V::LIGHT) {
      if (step >= g_first && step <= g_last) continue;   // left to the general pass
    }
    const int cwin = A0 - b0;             // workgroup window row t <-> lam = cwin - 63 + t
    const int lamlo = aw0 - b0 - 63, lamhi = aw0 + 31 - b0;
    // delta = i - j range of the wave tile
    const int dlo = DIR == 0 ? lamlo : -lamhi, dhi = DIR == 0 ? lamhi : -lamlo;
    bool wave_none = (b0 >= L) || (aw0 >= L);
    if (sh.wl >= 0 && dlo > sh.wl) wave_none = true;
    if (sh.wr >= 0 && -dhi > sh.wr) wave_none = true;
    const bool wave_full = (b0 + BOTH <= L) && (aw0 + WROWS <= L) &&
                           (sh.wl < 0 || dhi <= sh.wl) && (sh.wr < 0 || -dlo <= sh.wr);
    // ---- tile classes ----
    int rcls = 0, ccls = 0;   // 0 general, 1 = all end A, 2 = all end B
    bool wg_general = true;
    if constexpr (V::CLIP) {
      const int ta = V::TA(span), tb = V::TB(span);
      if constexpr (V::HAS_ROW && !V::DFAT) {
        if (lamhi <= ta) rcls = 1; else if (lamlo >= tb) rcls = 2;
      }
      if constexpr (V::HAS_COL && !V::DFAT) {
        if (-lamlo <= ta) ccls = 1; else if (-lamhi >= tb) ccls = 2;
      }
      wg_general = wg_gen(b0);
    }
    int acls = 0;            // ALiBi side of the diagonal: 1 every i >= j, 2 every i < j, 0 both
    bool lut_needed = true;  // ALiBi: some wave of the workgroup straddles the diagonal
    if constexpr (MECH == MECH_ALIBI) {
      if (dlo >= 0) acls = 1; else if (dhi < 0) acls = 2;
      const int wlo = DIR == 0 ? cwin - 63 : -(cwin + 127), whi = DIR == 0 ? cwin + 127 : -(cwin - 63);
      lut_needed = wlo < 0 && whi >= 0;
    }
    int t5cls = 0, t5b = 0;   // T5: one bucket for the whole wave tile, and which
    if constexpr (MECH == MECH_T5) {
      const int lo = clampi(dlo, 1 - L, L - 1), hi = clampi(dhi, 1 - L, L - 1);
      if (lo >= sh.t5sat) {            // past the last threshold: no map read
        t5cls = 1;
        t5b = sh.t5b_pos;
      } else if (hi <= -sh.t5sat) {
        t5cls = 1;
        t5b = sh.t5b_neg;
      } else {
        t5b = a.bucket[lo + L - 1];
        if ((lo >= 0 || hi < 0) && t5b == a.bucket[hi + L - 1]) t5cls = 1;
      }
    }

    // ---- stage ----
    __syncthreads();
    float tkl = 0.f, tkd = 0.f;   // (T-XL key side: LSE and D read with the tiles)
    if (V::TK && NP == 1 && step > 0) {
      // bf16 T-XL key side after the first step: the tiles, the 64 new column-window rows and
      // their v.r values in one branch-free block of reads (rows past L and window rows of no
      // table row read a valid row and store zeros)
      // (lane-derived values recomputed from an opaque thread index, not hoisted and spilled)
      int t = tid;
      asm volatile("" : "+v"(t));
      const int r = t >> 2, cc = (t & 3) * 16, ln = t & 63;
      const int yr = min(b0 + r, L - 1);
      const int wr = V::col_of((b0 - A0 - (BLANE - 1)) + 2 * BOTH + r, span, nrel, toff);
      const int vrr = V::col_of((b0 - A0 - (BLANE - 1)) + 2 * BOTH + ln, span, nrel, toff);
      // (bases rebuilt here from the kernel arguments in scalar registers, not hoisted and
      // spilled; the key side streams Q and dO, and its column-side table is rel_a)
      int hs = __builtin_amdgcn_readfirstlane(h), bhs = __builtin_amdgcn_readfirstlane(bh);
      asm volatile("" : "+s"(hs), "+s"(bhs));
      const int64_t sl = (int64_t)bhs * L * (2 * kHeadDim);
      const uint32_t oq = (uint32_t)(yr * (2 * kHeadDim) + 2 * cc);
      const uint32_t ow = (uint32_t)(max(wr, 0) * (2 * kHeadDim) + 2 * cc);
      gchar* gq = scalar_ptr(a.q) + sl + oq;
      gchar* go = scalar_ptr(a.dout) + sl + oq;
      gchar* gw = scalar_ptr(a.rel_a) + 2 * ((int64_t)hs * sh.rel_hs) + ow;
      typedef __attribute__((address_space(1))) const u32x4 gu4;
      u32x4 q0 = *(gu4*)gq, q1 = *(gu4*)(gq + 16), o0 = *(gu4*)go, o1 = *(gu4*)(go + 16);
      u32x4 w0 = *(gu4*)gw, w1 = *(gu4*)(gw + 16);
      const uint32_t ol = 4u * (uint32_t)min(b0 + ln, L - 1);
      float vr = load_f32(scalar_ptr(a.vr) + 4 * ((int64_t)hs * nrel), 4u * (uint32_t)max(vrr, 0));
      tkl = load_f32(scalar_ptr(a.lse) + 4 * ((int64_t)bhs * L), ol);
      tkd = load_f32(scalar_ptr(a.dsum) + 4 * ((int64_t)bhs * L), ol);
      // the previous step's leaving block, after this step's reads
      if constexpr (TK_DEFER) flush_r(rflush, b0 - BOTH);
      const u32x4 z = {0u, 0u, 0u, 0u};
      const bool yin = b0 + r < L, win_ok = wr >= 0;
      const int p0 = wrow(2 * BOTH, xrot);
      *(u32x4*)(ys + r * TSTR + cc) = yin ? q0 : z;
      *(u32x4*)(ys + r * TSTR + cc + 8) = yin ? q1 : z;
      *(u32x4*)(y2s + r * TSTR + cc) = yin ? o0 : z;
      *(u32x4*)(y2s + r * TSTR + cc + 8) = yin ? o1 : z;
      *(u32x4*)(win + (p0 + r) * TSTR + cc) = win_ok ? w0 : z;
      *(u32x4*)(win + (p0 + r) * TSTR + cc + 8) = win_ok ? w1 : z;
      if (tid < BOTH) *win_vec(win, p0 + tid) = vrr >= 0 ? vr : 0.f;
    } else if constexpr (V::TG1) {   // registers are the limit here: stage directly
      stage64<T, NP>(ys, yg, b0, L);
      stage64<T, NP>(y2s, y2g, b0, L);
    } else {
      py.store(ys);
      py2.store(y2s);
    }
    if constexpr (V::LUTP) {
      if (lut_needed && tid < WIN) vec_s[tid] = plut;
    }
    if constexpr (MECH == MECH_TXL && DIR == 0) {
      if (tid < BOTH) ovec_s[tid] = puk;   // (read one step ahead)
    }
    if constexpr (DIR == 1) {
      if (tid < BOTH) {
        // (read here when not prefetched: locals, so that nothing stays live across steps)
        float nl = pnl, nd = pdd;
        if (V::TK && NP == 1 && step > 0) {
          // LSE log2 e (+inf for rows past L or with no allowed key) and D, as lsd_vals gives
          const bool in = b0 + tid < L;
          nl = tkl * kLog2e;
          nl = (in && nl > kNegInf) ? nl : __builtin_inff();
          nd = in ? tkd : 0.f;
        } else if constexpr (!PF_LSD) {
          lsd_vals(b0, nl, nd);
        }
        lsd_s[tid] = nl;
        lsd_s[BOTH + tid] = nd;
        if constexpr (MECH == MECH_ALIBI) {
          ainit_s[tid] = ovec_s[tid] + nl;
          ainit_s[BOTH + tid] = ovec_s[BOTH + tid] + nl;
        }
      }
    }
    if constexpr (V::CLIP && V::HAS_COL && !V::DFAT) {
      // end A values of the 64 streamed rows, then end B: each a contiguous vector (key side:
      // plus -LSE / s, the score start of a column-clipped tile)
      const float nl = DIR == 1 ? pnl : 0.f;
      if (tid < BOTH) {
        ovec_s[tid] = pov[0] + nl;
        ovec_s[BOTH + tid] = pov[1] + nl;
      }
    }
    // row side staged now when there is no column side
    if constexpr (V::TQ) {
      // every T-XL tile is general; after the first step only rows 0..63 are new
      auto rowfn = [&](int x) { return V::row_of(cwin - 63 + x, span, nrel, toff); };
      if (step == 0) {
        stage_window<T, NP>(win, trow, rowfn);
        for (int x = tid; x < WIN; x += 256) {
          const int r = rowfn(x);
          *win_vec(win, x) = (r >= 0) ? a.vr[(int64_t)h * nrel + r] : 0.f;
        }
      } else {
        pwn.store_at(win, WIN * TSTR, xrot);
        if (tid < BOTH) *win_vec(win, xrot + tid) = pvr;
      }
    } else if constexpr (V::ROW && !V::COL) {
      if (wg_general) stage_window<T, NP>(win, trow, rowfn_at(b0));
    }
    // column side first (its window is replaced by the row-side window afterwards)
    if constexpr (V::TK) {
      // column window row x <-> mu = b - a = (b0 - A0 - 127) + x; after the first step only
      // rows 128..191 are new, at physical rows wrow(128, xrot) ..
      auto colfn = [&](int x) { return V::col_of((b0 - A0 - (BLANE - 1)) + x, span, nrel, toff); };
      if (step == 0) {
        stage_window<T, NP>(win, tcol, colfn);
        for (int x = tid; x < WIN; x += 256) {
          const int r = colfn(x);
          *win_vec(win, x) = (r >= 0) ? a.vr[(int64_t)h * nrel + r] : 0.f;
        }
      } else if constexpr (NP == 2) {   // (bf16: staged with the tiles above)
        const int p0 = wrow(2 * BOTH, xrot);
        stage_window_rows<T, NP>(win, tcol, colfn, 2 * BOTH, p0);
        if (tid < BOTH) {
          const int r = colfn(2 * BOTH + tid);
          *win_vec(win, p0 + tid) = (r >= 0) ? a.vr[(int64_t)h * nrel + r] : 0.f;
        }
      }
    } else if constexpr (V::COL) {
      if (wg_general) stage_window<T, NP>(win, tcol, colfn_at(b0));
    }
    // issue the next step's tile reads (after this step's staging reads have been consumed)
    next = step + 1;
    while (next < nsteps && step_skipped(next)) ++next;
    if (!V::TG1 && next < nsteps) {
      py.load(yg, step_base(next), L);
      py2.load(y2g, step_base(next), L);
    }
    if constexpr (ANY_PF) {
      if (next < nsteps) scalars_load(step_base(next));
    }
    if constexpr (V::TQ) {
      if (step + 1 < nsteps) {
        const int row0 = (cwin - BOTH) - 63 + toff;   // window rows 0..63 of the next step
        pwn.load_range(trow, row0, 0, nrel);
        if (tid < BOTH) {
          const int r = row0 + tid;
          pvr = (r >= 0 && r < nrel) ? a.vr[(int64_t)h * nrel + r] : 0.f;
          const int yy = b0 + BOTH + tid;
          puk = (yy < L) ? a.uk[(int64_t)bh * L + yy] : 0.f;
        }
      }
    }
    __syncthreads();

    f32x16 sc[2];
    Op<NP> yop[2][4];
    if (!wave_none) {
      if constexpr (KINIT) {
        // key side: the scores start from -LSE / s of each streamed query (plus the streamed
        // row's end-row constant on a column-clipped tile, or the ALiBi ramp on a one-sided
        // tile), so that P = exp2(c S + c lconst) takes one fma per element
        const float* iv = lsd_s;
        if constexpr (V::CLIP && V::HAS_COL) {
          if (ccls != 0) iv = ovec_s + (ccls == 1 ? 0 : BOTH);
        }
        if constexpr (MECH == MECH_ALIBI) {
          if (acls != 0) iv = ainit_s + (acls == 1 ? BOTH : 0);
        }
        other_dot_lane<NP, true>(sc, ys, xop, yop, iv);
      } else if constexpr (MECH == MECH_TXL && DIR == 0) {
        // T-XL query side: the scores start from u.k of each streamed key
        other_dot_lane<NP, true>(sc, ys, xop, yop, ovec_s);
      } else if constexpr (V::CLIP && V::HAS_COL) {
        // a column-clipped wave tile starts its scores from the end-row constant of each
        // streamed row
        if (ccls != 0) other_dot_lane<NP, true>(sc, ys, xop, yop, ovec_s + (ccls == 1 ? 0 : BOTH));
        else other_dot_lane<NP>(sc, ys, xop, yop);
      } else if constexpr (MECH == MECH_ALIBI) {
        // streamed-row ramp: +m y / s when the streamed rows are keys below the queries
        // (query side, i >= j) or queries above the keys (key side, i < j), else -m y / s
        const bool plus = (DIR == 0) == (acls == 1);
        if (acls != 0) other_dot_lane<NP, true>(sc, ys, xop, yop, ovec_s + (plus ? 0 : BOTH));
        else other_dot_lane<NP>(sc, ys, xop, yop);
      } else {
        other_dot_lane<NP>(sc, ys, xop, yop);
      }
    }
    float lconst = 0.f;   // per-lane additive term (y units)
    if constexpr (V::HAS_COL) {
      if (!wave_none) {
        if (V::CLIP && ccls != 0) {
          // already in the accumulator start
        } else if constexpr (V::TK) {
          col_skew_add<NP, true, true>(sc, win, (BLANE - WROWS) - WROWS * w, 0, ys, gs, xrot);
          col_skew_add<NP, true, true>(sc, win, (BLANE - WROWS) - WROWS * w, 1, ys, gs, xrot);
        } else if (V::COL && wg_general) {
          col_skew_add<NP, MECH == MECH_TXL>(sc, win, (BLANE - WROWS) - WROWS * w, 0, ys, gs);
          col_skew_add<NP, MECH == MECH_TXL>(sc, win, (BLANE - WROWS) - WROWS * w, 1, ys, gs);
        }
      }
    }
    if constexpr (V::ROW && V::COL) {
      if (wg_general) {
        __syncthreads();   // column-side window reads done
        stage_window<T, NP>(win, trow, rowfn_at(b0));
        __syncthreads();
      }
    }
    if constexpr (V::HAS_ROW) {
      if (!wave_none) {
        if (V::CLIP && rcls != 0) {
          lconst = (rcls == 1) ? rcA : rcB;
        } else if constexpr (V::ROW) {
          f32x16 g[3];
          if constexpr (V::TQ) row_products<NP, true, true>(g, win, WROWS * w, xop, xrot);
          else row_products<NP, MECH == MECH_TXL>(g, win, WROWS * w, xop);
          row_skew_add(sc, g, gs);
        }
      }
    }
    if constexpr (MECH == MECH_T5) {
      if (!wave_none) {
        if (t5cls == 1) {
          const int lo = clampi(DIR == 0 ? lamlo : -lamhi, 1 - L, L - 1);
          const int lamx = DIR == 0 ? lo : -lo;
          lconst = vec_s[lamx - (cwin - 63)];
        } else {
          add_offset_vec(sc, vec_s, WROWS * w);
        }
      }
    }
    if constexpr (MECH == MECH_TXL) {
      if (!wave_none) {
        if (DIR == 1) lconst = ukl;
      }
    }
    if constexpr (MECH == MECH_ALIBI) {
      if (!wave_none) {
        // lane-row term: -m (i - b0) / s or +m (i - b0) / s on the query side, the key side
        // mirrored (its lane rows are keys)
        const float da = am * (float)(my_a - b0);
        if (acls == 1) lconst = DIR == 0 ? -da : da;
        else if (acls == 2) lconst = DIR == 0 ? da : -da;
        else add_offset_vec(sc, vec_s, WROWS * w);
      }
    }

    f32x16 ds[2];
    Op<NP> dso[4];   // dS as bf16 MFMA operands (16 other-side rows each)
    if (!wave_none) {
      // dP first, its MFMAs run while the exponentials below are computed
      Op<NP> y2op[2][4];
      f32x16 dp[2];
      // dP starts from -D (the lane's on the query side, the streamed row's on the key side)
      if constexpr (DIR == 0) other_dot_lane_from<NP>(dp, y2s, x2op, y2op, -dsum_l);
      // the key side too, except where registers are the limit (general passes, T-XL)
      constexpr bool DP_FIRST = KINIT && !V::DFAT;
      if constexpr (DP_FIRST) other_dot_lane<NP, true>(dp, y2s, x2op, y2op, lsd_s + BOTH);
      // ---- P ----  (the key-side scores already hold -LSE / s, except in the T-XL pass)
      const float pbias = DIR == 0 ? lconst * c - lse2 : lconst * c;
      if constexpr (DIR == 1 && !KINIT) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *(const f32x4*)(lsd_s + 32 * b + 8 * g + 4 * kh);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sc[b][4 * g + i] = fast_exp2(fmaf(sc[b][4 * g + i], c, lconst * c - l4[i]));
          }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[b][r] = fast_exp2(fmaf(sc[b][r], c, pbias));
      }
      if (!wave_full) {
        const int wlx = sh.wl < 0 ? L : sh.wl, wrx = sh.wr < 0 ? L : sh.wr;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int y = 32 * b + 8 * (r >> 2) + 4 * kh + (r & 3);
            const int ii = DIR == 0 ? my_a : b0 + y;
            const int jj = DIR == 0 ? b0 + y : my_a;
            sc[b][r] = pair_ok(ii, jj, L, wlx, wrx) ? sc[b][r] : 0.f;
          }
      }
      if constexpr (KINIT && !DP_FIRST) other_dot_lane<NP, true>(dp, y2s, x2op, y2op, lsd_s + BOTH);
      else if constexpr (DIR == 1 && !KINIT) other_dot_lane<NP>(dp, y2s, x2op, y2op);
      // ---- dS = P (dP - D) ----
      if constexpr (DIR == 1 && !KINIT) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 d4 = *(const f32x4*)(lsd_s + BOTH + 32 * b + 8 * g + 4 * kh);
#pragma unroll
            for (int i = 0; i < 4; ++i) ds[b][4 * g + i] = sc[b][4 * g + i] * (dp[b][4 * g + i] - d4[i]);
          }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) ds[b][r] = sc[b][r] * dp[b][r];
      }
      if constexpr (MECH == MECH_TXL && DIR == 1) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) colsum += ds[b][r];
      }
      if constexpr (MECH == MECH_ALIBI && DIR == 0) {
        // |i - j| = (my_a - b0) - y below the diagonal, y - (my_a - b0) above, with y the
        // streamed row of the register (a constant plus 4 kh)
        const float di = (float)(my_a - b0);
        if (acls != 0) {
          float rs = 0.f, yw = 0.f;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              rs += ds[b][r];
              yw = fmaf((float)(32 * b + 8 * (r >> 2) + (r & 3)), ds[b][r], yw);
            }
          yw = fmaf((float)(4 * kh), rs, yw);
          amacc += (acls == 1) ? fmaf(di, rs, -yw) : fmaf(-di, rs, yw);
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float y = (float)(32 * b + 8 * (r >> 2) + 4 * kh + (r & 3));
              amacc = fmaf(fabsf(di - y), ds[b][r], amacc);
            }
        }
      }
      if constexpr (V::DFAT && V::HAS_ROW) {
        // row-side clipped elements: their dX_rel comes through the window's end rows, and
        // the end rows' table gradient needs their sums per lane row
        if (lamlo <= V::TA(span) || lamhi >= V::TB(span)) {
          // element y has lam = my_a - b0 - y: end A iff TA - lam = sa + y >= 0, end B iff
          // lam - TB = sb - y >= 0.  The tests are sign bits of integer sums (no lane masks:
          // the compiler would compute all 32 of a step at once and spill them)
          const int sa = V::TA(span) - (my_a - b0) + 4 * kh, sb = (my_a - b0) - V::TB(span) - 4 * kh;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int yc = 32 * b + 8 * (r >> 2) + (r & 3);   // y - 4 kh
              const uint32_t bits = __float_as_uint(ds[b][r]);
              cA += __uint_as_float(bits & ~(uint32_t)((sa + yc) >> 31));
              cB += __uint_as_float(bits & ~(uint32_t)((sb - yc) >> 31));
            }
          asm volatile("" : "+v"(cA), "+v"(cB));
        }
        // dS into the wave's buffer now (its skew reads are done), so that the fp32 copy dies
        // before the content gradients; the row-side dX_rel reads it back after them
        wave_lds_sync();
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 v4 = {ds[b][4 * g4], ds[b][4 * g4 + 1], ds[b][4 * g4 + 2], ds[b][4 * g4 + 3]};
            *(f32x4*)(gs + l32 * GS2 + 32 * b + 8 * g4 + 4 * kh) = v4;
          }
      }
      // ---- content gradients (P and dS packed to bf16 once; the fp32 copies can die) ----
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) dso[cc] = op_from_acc<NP>(ds, cc);
      if constexpr (DIR == 1) {
        Op<NP> po[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) po[cc] = op_from_acc<NP>(sc, cc);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            Op<NP> yt = op_rows_tr<NP>(y2s, BOTH * TSTR, TSTR, 16 * cc, 32 * db);
            mma<NP>(vacc[db], yt, po[cc]);
          }
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          Op<NP> yt = op_rows_tr<NP>(ys, BOTH * TSTR, TSTR, 16 * cc, 32 * db);
          mma<NP>(gacc[db], yt, dso[cc]);
        }
    }

    // ---- light pass: the whole wave tile reads one row-side end row ----
    if constexpr (V::CLIP && V::HAS_ROW && !V::DFAT) {
      if (!wave_none) {
        float tot = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) tot += ds[b][r];
        if (rcls == 1) cA += tot; else cB += tot;
      }
    }

    // ---- general pass (Shaw / DeBERTa): row-side dX_rel from the wave's dS buffer ----
    if constexpr (V::DFAT && V::HAS_ROW) {
      if (!wave_none) {
        wave_lds_sync();   // the wave's dS writes (before the content gradients) are visible
        // dX_rel^T[d][x] += sum_t Win[32 w + t][d] E[x][t], E[x][t] = dS[x][x + 63 - t] for t
        // in [x, x + 63] (else 0), read along the skewed diagonal of the buffer
        const float* grow = gs + l32 * GS2 + l32 + 63 - 4 * kh;
        // band tests against lq = l32 - 4 kh; lq is opaque to the compiler, so the tests are redone
        // each step (hoisted out of the step loop, their lane masks spill the scalar registers)
        int lq = l32 - 4 * kh;
        asm volatile("" : "+v"(lq));
#pragma unroll
        for (int cc = 0; cc < 6; ++cc) {
          float e8[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float v0 = grow[-(16 * cc + j)], v1 = grow[-(16 * cc + 8 + j)];
            if (cc < 2) { v0 = 16 * cc + j >= lq ? v0 : 0.f; v1 = 16 * cc + 8 + j >= lq ? v1 : 0.f; }
            if (cc > 3) {
              v0 = 16 * cc + j - 63 <= lq ? v0 : 0.f;
              v1 = 16 * cc + 8 + j - 63 <= lq ? v1 : 0.f;
            }
            e8[j] = v0;
            e8[4 + j] = v1;
          }
          Op<NP> eop = op_from_f32<NP>(e8);
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            Op<NP> wt = op_rows_tr<NP>(win, WIN * TSTR, TSTR, WROWS * w + 16 * cc, 32 * db);
            mma<NP>(gacc[db], wt, eop);
          }
        }
      }
    }

    // ---- T-XL key side (and DeBERTa general pass): table GEMM over the streamed rows ----
    if constexpr (V::TG1) {
      // E2T[y][t] = dS[y][x] with t = y - x + 127, in the column-skew buffer's space: for one
      // register, the 32 lanes of a half-wave write 32 consecutive t
      uint16_t* e2t = (uint16_t*)gsb;   // NP planes of [BOTH][ESTRT]
      if (wave_none) {   // a wave with no pairs contributes zeros (wave-uniform)
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) dso[cc].p[pl] = u4_to_bf8(z);
      }
      __syncthreads();   // every wave's column-skew reads are done
      // The band covers t in [y, y + 127] of row y; every other entry of the 192 columns the
      // GEMM reads must be zero.  The rows are cleared whole (six 16-byte stores per thread and
      // plane) before the band is written, so the GEMM's edge chunks need no per-element masks.
      {
        const u32x4 z = {0u, 0u, 0u, 0u};
        uint16_t* zr = e2t + (tid >> 2) * ESTRT + 48 * (tid & 3);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
          for (int q = 0; q < 6; ++q) *(u32x4*)(zr + pl * BOTH * ESTRT + 8 * q) = z;
      }
      __syncthreads();
      uint16_t* eb = e2t + (127 - (WROWS * w + l32) + 4 * kh) + 4 * kh * ESTRT;
#pragma unroll
      for (int pl = 0; pl < NP; ++pl)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          // operand slot i of dso[cc] is register 8 (cc % 2) + i of block cc / 2
          const u32x4 wv = __builtin_bit_cast(u32x4, dso[cc].p[pl]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * (cc & 1) + i;
            const int yc = 32 * (cc >> 1) + 8 * (r >> 2) + (r & 3);   // y - 4 kh
            const uint32_t word = wv[i >> 1];
            eb[pl * BOTH * ESTRT + yc * (ESTRT + 1)] =
                (uint16_t)((i & 1) ? (word >> 16) : (word & 0xFFFFu));
          }
        }
      __syncthreads();
      if constexpr (V::TK) {
        // (chunk-outer: each streamed-row operand is read once for the three blocks; every
        // accumulator still takes its chunks in ascending order.  The general passes of Shaw
        // and DeBERTa, tighter on registers, keep the block-outer order below.)
#pragma unroll
        for (int cq = 0; cq < 4; ++cq) {
          const int ylo = 16 * cq, yhi = ylo + 15;
          Op<NP> qop2 = op_rows_tr<NP>(ys, BOTH * TSTR, TSTR, ylo, 32 * gdb);
#pragma unroll
          for (int i = 0; i < 3; ++i) {
            const int ab = gp + 2 * i;
            const int tlo = 32 * ab, thi = tlo + 31;
            if (thi < ylo || tlo > yhi + 127) continue;   // no pair of this block and chunk
            Op<NP> eop = op_rows_tr<NP>(e2t, BOTH * ESTRT, ESTRT, ylo, tlo);
            mma<NP>(racc[i], eop, qop2);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const int ab = gp + 2 * i;
          const int tlo = 32 * ab, thi = tlo + 31;
#pragma unroll
          for (int cq = 0; cq < 4; ++cq) {
            const int ylo = 16 * cq, yhi = ylo + 15;
            if (thi < ylo || tlo > yhi + 127) continue;   // no pair of this block and chunk
            Op<NP> eop = op_rows_tr<NP>(e2t, BOTH * ESTRT, ESTRT, ylo, tlo);
            Op<NP> qop2 = op_rows_tr<NP>(ys, BOTH * TSTR, TSTR, ylo, 32 * gdb);
            mma<NP>(racc[i], eop, qop2);
          }
        }
      }
      // block gp leaves the window with this step (the next window starts 64 offsets higher)
      if constexpr (TK_DEFER) {
        rflush = racc[0];   // written early in the next step (or after the sweep)
      } else if constexpr (V::TK) {
        flush_r(racc[0], b0);
      } else {
        flush_col(racc[0], b0 - A0 - (BLANE - 1) + 32 * gp + 4 * kh);
      }
      racc[0] = racc[1];
      racc[1] = racc[2];
      racc[2] = f32x16{};
    }

    // ---- per-offset fp32 sums of dS (T5 bias gradient; T-XL v term and v gradient) ----
    if constexpr (V::DIAG) {
      const bool single = (MECH == MECH_T5) && t5cls == 1;
      // lane l: sums[0] = diagonal t = l, sums[1] = diagonal t = l + 64 (l < 32)
      float sums[2] = {0.f, 0.f};
      if (!wave_none && !single) {
        // dS[n][y] into the wave buffer, then sums along the diagonals t = n - y + 63
        wave_lds_sync();
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 v4 = {ds[b][4 * g4], ds[b][4 * g4 + 1], ds[b][4 * g4 + 2], ds[b][4 * g4 + 3]};
            *(f32x4*)(gs + l32 * GS2 + 32 * b + 8 * g4 + 4 * kh) = v4;
          }
        wave_lds_sync();
        if constexpr (V::GSREL) {
          // dX_rel^T[d][x] += sum_t Win[32 w + t][d] E[x][t] with E[x][t] = dS[x][x + 63 - t]
          // for t in [x, x + 63] (else 0), read along the skewed diagonal of the buffer
          const float* grow = gs + l32 * GS2 + l32 + 63 - 4 * kh;
          // band tests against lq = l32 - 4 kh; lq is opaque to the compiler, so the tests are redone
          // each step (hoisted out of the step loop, their lane masks spill the scalar registers)
          int lq = l32 - 4 * kh;
          asm volatile("" : "+v"(lq));
#pragma unroll
          for (int cc = 0; cc < 6; ++cc) {
            float e8[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float v0 = grow[-(16 * cc + j)], v1 = grow[-(16 * cc + 8 + j)];
              if (cc < 2) { v0 = 16 * cc + j >= lq ? v0 : 0.f; v1 = 16 * cc + 8 + j >= lq ? v1 : 0.f; }
              if (cc > 3) {
                v0 = 16 * cc + j - 63 <= lq ? v0 : 0.f;
                v1 = 16 * cc + 8 + j - 63 <= lq ? v1 : 0.f;
              }
              e8[j] = v0;
              e8[4 + j] = v1;
            }
            Op<NP> eop = op_from_f32<NP>(e8);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
              Op<NP> wt = op_rows_tr_rot<NP>(win, WIN * TSTR, TSTR, WROWS * w + 16 * cc, 32 * db,
                                             xrot);
              mma<NP>(gacc[db], wt, eop);
            }
          }
        }
        if constexpr (MECH == MECH_TXL) {
          // Lane l sums diagonal t = l (rows 0 .. min(l, 31)) and, for l < 32, diagonal
          // t = l + 64 (rows l + 1 .. 31): one element of every row, rows in ascending order,
          // so the 32 reads are independent and issue back to back (every T-XL tile runs this)
          // One running sum over the rows; its value after row min(l, 31) is diagonal l's sum
          // and the rest of it diagonal l + 64's.
          const float* gd = gs + (63 - lane);   // row n of diagonal l: gd[n * GS2 + n]
          int ln = lane;   // opaque: the tests n <= lane are redone each step, not hoisted
          asm volatile("" : "+v"(ln));
          float run = 0.f, pre = 0.f;
#pragma unroll
          for (int n = 0; n < WROWS; ++n) {
            const bool first = n <= ln;
            run += gd[n * GS2 + n - (first ? 0 : 64)];
            pre = first ? run : pre;
          }
          sums[0] = pre;
          sums[1] = run - pre;
        } else {
          // T5 reaches this only on its multi-bucket tiles: the compact loop, same order
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int t = lane + 64 * half;
            if (t < 96) {
              // diagonal t runs through rows n with 0 <= n + 63 - t < 64
              const int n0 = max(0, t - 63), n1 = min(WROWS - 1, t);
              float sum = 0.f;
              for (int n = n0; n <= n1; ++n) sum += gs[n * GS2 + n + 63 - t];
              sums[half] = sum;
            }
          }
        }
      } else if constexpr (V::T5BIN) {
        // single bucket (T5 only): the tile's dS joins this lane's running sum of its bucket
        if (!wave_none) {
          const int bk = __builtin_amdgcn_readfirstlane(t5b);   // (wave-uniform)
          if (bk != t5cur) {
            t5_flush();
            t5cur = bk;
          }
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) t5acc += ds[b][r];
        }
      }
      if constexpr (V::T5BIN) {
        // Multi-bucket tile: the diagonal sums join their buckets' sums.  Diagonal t holds
        // offset i - j = aw0 - b0 - 63 + t, and every bucket is one run of consecutive offsets
        // (the bucket grows with |i - j| on each side of the diagonal), so a segmented scan
        // over the lanes in a fixed order sums each run and the run's last lane adds it.
        if (!wave_none && !single) {
          const int dbase = aw0 - b0 - 63;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int t = lane + 64 * half;
            const bool valid = t < 96;   // (offsets past the sequence hold dS = 0)
            const int bk = valid ? a.bucket[clampi(dbase + t, 1 - L, L - 1) + L - 1] : -1;
            float x = valid ? sums[half] : 0.f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
              const float xu = __shfl_up(x, o);
              const int bu = __shfl_up(bk, o);
              if (lane >= o && bu == bk) x += xu;
            }
            const int bn = __shfl_down(bk, 1);
            if (valid && (lane == 63 || bn != bk)) binw[bk] += x;
          }
        }
      } else {
        // Diagonal t of this step is diagonal t + 64 of the next for t < 32: lanes 0..31 carry
        // sums[0] into their next sums[1]; the wave's 64 offsets t = 32 .. 95 are final (lane
        // 32 + i: t = 32 + i from sums[0]; lane i: t = 64 + i from sums[1] and the carry), and
        // after the last step also t = 0 .. 31.  No workgroup barrier: each wave writes its own
        // partial.
        const float fin = (lane >= 32) ? sums[0] : sums[1] + dcarry;
        dcarry = (lane < 32) ? sums[0] : 0.f;
        float* pw = pdiag + w * ndg + (aw0 - b0 - 63) - (lam_base + 32 * w) - dxo;
        pw[(lane >= 32) ? lane : 64 + lane] = fin;
        if (step == nsteps - 1 && lane < 32) pw[lane] = dcarry;
      }
    }
  }

  // ---- T5: this workgroup's bucket sums of dS, the waves in a fixed order ----
  if constexpr (V::T5BIN) {
    t5_flush();
    __syncthreads();
    const int nbk = sh.nbk;
    for (int k = tid; k < nbk; k += 256)
      a.part_qv[owner * nbk + k] = (bins_s[k] + bins_s[kMaxBuckets + k]) +
                                   (bins_s[2 * kMaxBuckets + k] + bins_s[3 * kMaxBuckets + k]);
  }

  // ---- ALiBi: this workgroup's share of sum dS |i - j|, in a fixed order ----
  if constexpr (MECH == MECH_ALIBI && DIR == 0) {
    float t = amacc + xhalf(amacc);
    for (int m = 1; m < 32; m <<= 1) t += __shfl_xor(t, m);
    if (lane == 0) red_s[w] = t;
    __syncthreads();
    if (tid == 0) a.part_qv[owner] = (red_s[0] + red_s[1]) + (red_s[2] + red_s[3]);
  }

  // ---- final flush of the window accumulators ----
  if constexpr (V::DFAT && V::HAS_COL) {
    // blocks gp + 2 and gp + 4 of the last window (shifted into racc[0], racc[1])
    if (nsteps > 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) flush_col(racc[i], bt_last - A0 - (BLANE - 1) + 32 * (gp + 2 + 2 * i) + 4 * kh);
    }
  }
  if constexpr (V::TK) {
    // the last step's leaving block (still pending when deferred), then blocks gp + 2 and
    // gp + 4 of the last window (shifted into racc[0], racc[1]), which would have left with
    // the steps after it
    if (nsteps > 0) {
      if constexpr (TK_DEFER) flush_r(rflush, bt_last);
      flush_r(racc[0], bt_last + BOTH);
      flush_r(racc[1], bt_last + 2 * BOTH);
    }
  }

  // ---- light pass: hand the partial sums to the general pass ----
  if constexpr (V::LIGHT) {
    if constexpr (V::HAS_ROW) {
      cA += xhalf(cA);
      cB += xhalf(cB);
    }
    if (my_a < L) {
      const int64_t rowoff = ((int64_t)bh * L + my_a) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * db + 8 * g + 4 * kh;
          f32x4 v4 = {gacc[db][4 * g], gacc[db][4 * g + 1], gacc[db][4 * g + 2], gacc[db][4 * g + 3]};
          *(f32x4*)(a.xpart + rowoff + d) = v4;
          if constexpr (DIR == 1) {
            f32x4 w4 = {vacc[db][4 * g], vacc[db][4 * g + 1], vacc[db][4 * g + 2], vacc[db][4 * g + 3]};
            *(f32x4*)(a.vpart + rowoff + d) = w4;
          }
        }
      if (V::HAS_ROW && kh == 0) {
        a.cab[((int64_t)bh * L + my_a) * 2 + 0] = cA;
        a.cab[((int64_t)bh * L + my_a) * 2 + 1] = cB;
      }
    }
    return;
  }
  if constexpr (V::FAT) {
    if (my_a < L) {
      const int64_t rowoff = ((int64_t)bh * L + my_a) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * db + 8 * g + 4 * kh;
          f32x4 v4 = *(const f32x4*)(a.xpart + rowoff + d);
#pragma unroll
          for (int i = 0; i < 4; ++i) gacc[db][4 * g + i] += v4[i];
          if constexpr (DIR == 1) {
            f32x4 w4 = *(const f32x4*)(a.vpart + rowoff + d);
#pragma unroll
            for (int i = 0; i < 4; ++i) vacc[db][4 * g + i] += w4[i];
          }
        }
    }
  }

  // ---- end rows (clipped offsets): table gradient and lane gradient ----
  if constexpr (V::DFAT && V::ROW) {
    // cA / cB hold this lane's sum over its half of the other rows (this pass's clipped
    // elements, whose dX_rel came through the window); the light pass's sums still owe their
    // dX term
    cA += xhalf(cA);
    cB += xhalf(cB);
    float lA = 0.f, lB = 0.f;
    if (my_a < L) {
      lA = a.cab[((int64_t)bh * L + my_a) * 2 + 0];
      lB = a.cab[((int64_t)bh * L + my_a) * 2 + 1];
    }
    // end rows of the row-side table: sum over the lane rows of (cA + lA) X, with the lane rows
    // and the sums staged in the (now free) dS buffers
    float* ends = gsb;                                   // [2][BLANE]
    // lane rows X: two 64-row tiles of NP planes each, [2][NP][BOTH][TSTR]
    uint16_t* xst = (uint16_t*)(gsb + 2 * BLANE);
    __syncthreads();
    stage64<T, NP>(xst, xg, A0, L);
    stage64<T, NP>(xst + NP * BOTH * TSTR, xg, A0 + BOTH, L);
    if (kh == 0) {
      ends[WROWS * w + l32] = (my_a < L) ? cA + lA : 0.f;
      ends[BLANE + WROWS * w + l32] = (my_a < L) ? cB + lB : 0.f;
    }
    __syncthreads();
    if (tid < 2 * kHeadDim) {
      const int e = tid / kHeadDim, d = tid % kHeadDim;
      float acc = 0.f;
      for (int x = 0; x < BLANE; ++x) {
        const uint16_t* xr = xst + (x >> 6) * NP * BOTH * TSTR + (x & 63) * TSTR + d;
        float xv = bf_bits2f(xr[0]);
        if constexpr (NP == 2) xv += bf_bits2f(xr[BOTH * TSTR]);   // hi + lo: the fp32 value
        acc = fmaf(ends[e * BLANE + x], xv, acc);
      }
      const int row = e == 0 ? V::rowA(span) : V::rowB(span);
      float* f = prow + (int64_t)row * kHeadDim + d;
      *f = first ? acc : *f + acc;
    }
    // dX += lA T[rowA] + lB T[rowB]
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * db + 8 * (r >> 2) + 4 * kh + (r & 3);
        const float ta = Elem<T>::to_f(trow[(int64_t)V::rowA(span) * kHeadDim + d]);
        const float tb = Elem<T>::to_f(trow[(int64_t)V::rowB(span) * kHeadDim + d]);
        gacc[db][r] = fmaf(lA, ta, fmaf(lB, tb, gacc[db][r]));
      }
  }

  // ---- T-XL key side: dK += u * colsum; du partial = sum_j colsum_j k_j ----
  if constexpr (MECH == MECH_TXL && DIR == 1) {
    colsum += xhalf(colsum);
    const float* u = a.bias_a + (int64_t)h * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * db + 8 * (r >> 2) + 4 * kh + (r & 3);
        gacc[db][r] = fmaf(colsum, u[d], gacc[db][r]);
      }
    float* csum = lsd_s;   // the per-query vectors are dead after the sweep
    __syncthreads();
    if (kh == 0) csum[WROWS * w + l32] = (my_a < L) ? colsum : 0.f;
    __syncthreads();
    if (tid < kHeadDim) {
      // (rows past L read row L - 1 and meet a zero column sum: no early exit, so the reads
      // of each group of 16 rows are issued together instead of one round trip per row)
      float acc = 0.f;
      for (int x0 = 0; x0 < BLANE; x0 += 16) {
        float kv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          kv[j] = Elem<T>::to_f(xg[(int64_t)min(A0 + x0 + j, L - 1) * kHeadDim + tid]);
#pragma unroll
        for (int j = 0; j < 16; ++j) acc = fmaf(csum[x0 + j], kv[j], acc);
      }
      a.part_kv[((int64_t)bh * nb + bid % nb) * kHeadDim + tid] = acc;   // per slice
    }
  }

  // ---- store dX (dQ or dK) and dV ----
  if (my_a < L) {
    T* gx = (T*)(DIR == 0 ? a.dq : a.dk) + bh_off + (int64_t)my_a * kHeadDim;
    T* gv = (T*)a.dv + bh_off + (int64_t)my_a * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * kh;
        if constexpr (NP == 1) {
          u32x2 pk = {pack_bf16x2(gacc[db][4 * g] * s, gacc[db][4 * g + 1] * s),
                      pack_bf16x2(gacc[db][4 * g + 2] * s, gacc[db][4 * g + 3] * s)};
          *(u32x2*)(gx + d) = pk;
          if constexpr (DIR == 1) {
            u32x2 pv = {pack_bf16x2(vacc[db][4 * g], vacc[db][4 * g + 1]),
                        pack_bf16x2(vacc[db][4 * g + 2], vacc[db][4 * g + 3])};
            *(u32x2*)(gv + d) = pv;
          }
        } else {
          f32x4 v4 = {gacc[db][4 * g] * s, gacc[db][4 * g + 1] * s, gacc[db][4 * g + 2] * s,
                      gacc[db][4 * g + 3] * s};
          *(f32x4*)(gx + d) = v4;
          if constexpr (DIR == 1) {
            f32x4 w4 = {vacc[db][4 * g], vacc[db][4 * g + 1], vacc[db][4 * g + 2], vacc[db][4 * g + 3]};
            *(f32x4*)(gv + d) = w4;
          }
        }
      }
  }
}

// Every bf16 variant fits two workgroups per CU (LDS at most 80 KiB) and is compiled for two
// waves per SIMD (at most 256 registers per lane).  The fp32 variants hold two bf16 planes of
// every tile (at most 144 KiB of LDS) and run one workgroup per CU.
template <typename T, int MECH, int DIR, int PART, int FIRSTK = -1>
__global__ __launch_bounds__(256, Elem<T>::NP == 1 ? 2 : 1) void bwd_kernel(BwdArgs a) {
  bwd_body<T, MECH, DIR, PART, FIRSTK>(a);
}
}  // namespace relpos
