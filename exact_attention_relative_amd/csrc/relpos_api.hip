// C ABI: descriptor validation, workspace layout, T5 bucket thresholds and kernel dispatch.
#include <math.h>
#include <string.h>

#include <vector>

#include "../../include/relpos_attn.h"
#include <algorithm>

#include "relpos_kernels.h"

using namespace relpos;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kGroupWorkgroups = 512;   // one wave of workgroups: 2 per CU x 256 CUs
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------------ exact T5 thresholds
// Non-negative big integers, little-endian 32-bit limbs.
struct Big {
  std::vector<uint32_t> d{1u};
  void mul(uint32_t m) {
    uint64_t carry = 0;
    for (auto& x : d) {
      uint64_t v = (uint64_t)x * m + carry;
      x = (uint32_t)v;
      carry = v >> 32;
    }
    if (carry) d.push_back((uint32_t)carry);
  }
};
int cmp(const Big& a, const Big& b) {
  size_t na = a.d.size(), nb = b.d.size();
  while (na > 1 && a.d[na - 1] == 0) --na;
  while (nb > 1 && b.d[nb - 1] == 0) --nb;
  if (na != nb) return na < nb ? -1 : 1;
  for (size_t i = na; i-- > 0;)
    if (a.d[i] != b.d[i]) return a.d[i] < b.d[i] ? -1 : 1;
  return 0;
}
Big bigpow_prod(uint32_t x, int ex, uint32_t y, int ey) {
  Big r;
  for (int i = 0; i < ex; ++i) r.mul(x);
  for (int i = 0; i < ey; ++i) r.mul(y);
  return r;
}
// floor(ln(n / me) / ln(md / me) * E) >= t  <=>  n^E me^t >= md^t me^E
bool reaches(uint32_t n, int t, uint32_t me, uint32_t md, int E) {
  return cmp(bigpow_prod(n, E, me, t), bigpow_prod(md, t, me, E)) >= 0;
}

bool build_t5_map(const relpos_desc* d, T5Map* m) {
  memset(m, 0, sizeof(*m));
  const int nb = d->num_buckets;
  m->bidirectional = d->bidirectional ? 1 : 0;
  const int half = m->bidirectional ? nb / 2 : nb;
  m->half = half;
  m->max_exact = half / 2;
  const int E = half - m->max_exact;
  m->nthr = E - 1;
  if (m->nthr > kMaxThresholds) return false;
  const uint32_t me = (uint32_t)m->max_exact, md = (uint32_t)d->max_distance;
  for (int t = 1; t <= E - 1; ++t) {
    // smallest n in [me, md] with floor(...) >= t (n = md always reaches t <= E)
    uint32_t lo = me, hi = md;
    while (lo < hi) {
      uint32_t mid = lo + (hi - lo) / 2;
      if (reaches(mid, t, me, md, E)) hi = mid; else lo = mid + 1;
    }
    m->thr[t - 1] = (int)lo;
  }
  return true;
}

// ------------------------------------------------------------------ validation
struct Plan {
  bool fp32;
  int B, H, L;
  int nrel, txl_off;
  float scale;
  T5Map t5;
  // workspace offsets (bytes)
  size_t off_bucket, off_lut, off_rowc, off_keyc, off_uk, off_vr, off_dsum;
  size_t off_part_q, off_part_k, off_part_qv, off_part_kv, off_diag, off_xpart, off_vpart, off_cab;
  int64_t part_q_stride, part_k_stride;
  int nb, nrt, owners;
  int txl_group;   // T-XL key-side pass under max_partial_bytes: (batch, head) slices per group
  int fold;        // folded passes: batch entries (or slices, fold_slices) per partial slot
  bool fold_slices;  // Shaw / DeBERTa with one table for every head: fold (batch, head) slices
  int fold_owners; // their partial slots: ceil(B / fold) H nb
  int64_t rel_rows;   // rows of each relation table (0 for T5 / ALiBi)
  int64_t rel_hs;     // elements between the relation tables of consecutive heads (0 = shared)
  size_t fwd_bytes, bwd_bytes;
};

int make_plan(const relpos_desc* d, Plan* p) {
  if (!d) return RELPOS_E_INVALID;
  if (d->mech < RELPOS_T5 || d->mech > RELPOS_ALIBI) return RELPOS_E_INVALID;
  if (d->dtype != RELPOS_BF16 && d->dtype != RELPOS_FP32) return RELPOS_E_INVALID;
  if (d->batch < 0 || d->heads < 1 || d->seqlen < 0 || d->head_dim < 1) return RELPOS_E_INVALID;
  if (d->window_left < -1 || d->window_right < -1) return RELPOS_E_INVALID;
  if (!(isfinite(d->scale)) || d->scale < 0.f) return RELPOS_E_INVALID;
  if (d->max_partial_bytes < 0) return RELPOS_E_INVALID;
  if (d->head_dim != kHeadDim) return RELPOS_E_UNSUPPORTED;
  if (d->seqlen > (1 << 28) || d->heads > (1 << 20) || d->batch > (1 << 20)) return RELPOS_E_UNSUPPORTED;
  const int64_t nqb = (d->seqlen + 127) / 128;
  if (d->batch * d->heads * nqb > 0x7FFFFFFFLL) return RELPOS_E_UNSUPPORTED;
  memset(p, 0, sizeof(*p));
  p->fp32 = d->dtype == RELPOS_FP32;
  p->B = (int)d->batch;
  p->H = (int)d->heads;
  p->L = (int)d->seqlen;
  const int L = p->L;
  switch (d->mech) {
    case RELPOS_T5: {
      if (d->num_buckets < 2 || d->num_buckets > kMaxBuckets) return RELPOS_E_INVALID;
      if (d->bidirectional && (d->num_buckets % 2 != 0 || d->num_buckets < 4)) return RELPOS_E_INVALID;
      const int half = d->bidirectional ? d->num_buckets / 2 : d->num_buckets;
      if (half / 2 < 1 || d->max_distance <= half / 2) return RELPOS_E_INVALID;
      if (!build_t5_map(d, &p->t5)) return RELPOS_E_UNSUPPORTED;
      break;
    }
    case RELPOS_SHAW:
    case RELPOS_DEBERTA:
      if (d->rel_span < 1 || d->rel_span > (1 << 26)) return RELPOS_E_INVALID;
      break;
    case RELPOS_TXL:
    case RELPOS_ALIBI:
      break;
  }
  p->nrel = (d->window_right == 0) ? L : 2 * L - 1;
  if (p->nrel < 0) p->nrel = 0;
  p->txl_off = (d->window_right == 0) ? 0 : L - 1;
  // relation tables: rows per table, and one table per head or one shared by every head
  if (d->rel_head_stride < 0) return RELPOS_E_INVALID;
  switch (d->mech) {
    case RELPOS_SHAW: p->rel_rows = 2 * (int64_t)d->rel_span + 1; break;
    case RELPOS_DEBERTA: p->rel_rows = 2 * (int64_t)d->rel_span; break;
    case RELPOS_TXL: p->rel_rows = p->nrel; break;
    default: p->rel_rows = 0; break;
  }
  p->rel_hs = p->rel_rows > 0 ? d->rel_head_stride : 0;
  if (p->rel_hs != 0 && (p->rel_hs < p->rel_rows * kHeadDim || p->rel_hs % 8 != 0))
    return RELPOS_E_INVALID;
  // the kernels address rows inside one (batch, head) slice and inside one head's table with
  // 32-bit byte offsets
  {
    const int64_t esz = p->fp32 ? 4 : 2;
    const int64_t rows_max = std::max<int64_t>(L, p->rel_rows);
    if (rows_max * kHeadDim * esz >= ((int64_t)1 << 32)) return RELPOS_E_UNSUPPORTED;
  }
  if (d->scale > 0.f) p->scale = d->scale;
  else p->scale = (float)(1.0 / sqrt((d->mech == RELPOS_DEBERTA ? 3.0 : 1.0) * (double)d->head_dim));

  // ---- workspace layout ----
  const size_t rows = (size_t)p->B * p->H * L;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  const bool lut_path = d->mech == RELPOS_T5 || d->mech == RELPOS_ALIBI;
  if (lut_path) {
    p->off_bucket = take(sizeof(int32_t) * (size_t)(L > 0 ? 2 * L - 1 : 1));
    p->off_lut = take(sizeof(float) * (size_t)p->H * (L > 0 ? 2 * L - 1 : 1));
  }
  if (d->mech == RELPOS_SHAW || d->mech == RELPOS_DEBERTA) p->off_rowc = take(sizeof(float) * rows * 2);
  if (d->mech == RELPOS_DEBERTA) p->off_keyc = take(sizeof(float) * rows * 2);
  if (d->mech == RELPOS_TXL) {
    p->off_uk = take(sizeof(float) * rows);
    p->off_vr = take(sizeof(float) * (size_t)p->H * p->nrel);
  }
  p->fwd_bytes = off;
  // backward: D, per-workgroup partials (one owner per 128-row block of each (batch, head)),
  // and the per-head diagonal sums of the aggregation pass
  p->off_dsum = take(sizeof(float) * rows);
  p->nb = (L + 127) / 128;
  p->nrt = L + 256;
  p->owners = p->B * p->H * p->nb;
  const size_t own = (size_t)p->owners;
  // Shaw / DeBERTa general passes and the T-XL key-side pass: the batch entries of a head run
  // as `fold` consecutive launches into one partial slot.  The fewest groups of batch entries
  // that still give one full wave of workgroups (two per compute unit on 256 compute units); no
  // folding below that.  T-XL folds only when one batch entry gives at most one wave and no
  // max_partial_bytes is set; otherwise it runs slice groups (below).
  const bool txl_fold = d->mech == RELPOS_TXL && d->max_partial_bytes == 0 &&
                        (int64_t)p->H * p->nb <= kGroupWorkgroups;
  // A table that every head shares (Shaw / DeBERTa with rel_head_stride 0) folds whole
  // (batch, head) slices the same way, so that even one long batch entry shares its slots.
  p->fold = 1;
  p->fold_slices = (d->mech == RELPOS_SHAW || d->mech == RELPOS_DEBERTA) && p->rel_hs == 0;
  if (d->mech == RELPOS_SHAW || d->mech == RELPOS_DEBERTA || txl_fold) {
    const int units = p->fold_slices ? p->B * p->H : p->B;                        // what folds
    const int64_t per_unit = p->fold_slices ? p->nb : (int64_t)p->H * p->nb;      // its workgroups
    for (int ng = 1; ng <= units; ++ng) {
      if (ng * per_unit >= kGroupWorkgroups) {
        p->fold = (units + ng - 1) / ng;
        break;
      }
    }
  }
  p->fold_owners = p->fold_slices ? (p->B * p->H + p->fold - 1) / p->fold * p->nb
                                  : (p->B + p->fold - 1) / p->fold * p->H * p->nb;
  const int k = d->rel_span;
  if (d->mech == RELPOS_SHAW) p->part_q_stride = (int64_t)(2 * k + 1) * kHeadDim;
  if (d->mech == RELPOS_DEBERTA) p->part_q_stride = p->part_k_stride = (int64_t)(2 * k) * kHeadDim;
  if (d->mech == RELPOS_TXL) {
    // key-side r partial: rows for every offset, or with a two-sided window only the rows of
    // the owner's sweep (at most wl + wr + 382)
    int64_t rows_k = p->nrt;
    if (d->window_left >= 0 && d->window_right >= 0) {
      const int64_t wrows = ((int64_t)d->window_left + d->window_right + 382 + 63) / 64 * 64;
      rows_k = std::min<int64_t>(rows_k, wrows);
    }
    p->part_q_stride = rows_k * kHeadDim;
    // Folded (above), the partials hold ceil(B / fold) H slices.  Otherwise the (batch, head)
    // slices run in groups, each group's partials aggregated before the next reuses them: as
    // many slices as give one wave of workgroups, or, under max_partial_bytes, as fit in it (at
    // least one slice either way).
    const int64_t per_slice = (int64_t)p->nb * p->part_q_stride * (int64_t)sizeof(float);
    const int64_t nbh = (int64_t)p->B * p->H;
    const int64_t group = d->max_partial_bytes > 0
                              ? d->max_partial_bytes / std::max<int64_t>(per_slice, 1)
                              : kGroupWorkgroups / std::max<int64_t>(p->nb, 1);
    p->txl_group = txl_fold ? 0 : (int)std::max<int64_t>(1, std::min<int64_t>(nbh, group));
  }
  if (d->mech == RELPOS_TXL) {
    const size_t slots = p->txl_group > 0 ? (size_t)p->txl_group * p->nb : (size_t)p->fold_owners;
    p->off_part_q = take(sizeof(float) * slots * p->part_q_stride);
  } else if (p->part_q_stride) {
    p->off_part_q = take(sizeof(float) * (size_t)p->fold_owners * p->part_q_stride);
  }
  if (p->part_k_stride) p->off_part_k = take(sizeof(float) * (size_t)p->fold_owners * p->part_k_stride);
  if (d->mech == RELPOS_TXL) {
    // T-XL: per-offset sums, one partial row per wave of each query-side owner
    p->off_part_qv = take(sizeof(float) * own * diag_width(L, d->window_left, d->window_right) * 4);
    p->off_diag = take(sizeof(float) * (size_t)p->H * (L > 0 ? 2 * L - 1 : 1));
  }
  // T5: the bucket sums of each query-side owner; ALiBi: one slope sum per owner
  if (d->mech == RELPOS_T5) p->off_part_qv = take(sizeof(float) * own * d->num_buckets);
  if (d->mech == RELPOS_ALIBI) p->off_part_qv = take(sizeof(float) * own);
  if (d->mech == RELPOS_TXL) p->off_part_kv = take(sizeof(float) * own * kHeadDim);
  if (d->mech == RELPOS_SHAW || d->mech == RELPOS_DEBERTA) {
    // split passes: clipped-step partials handed from the light kernel to the general one
    // (dX, the end-row sums, and dV on the key side)
    p->off_xpart = take(sizeof(float) * rows * kHeadDim);
    p->off_cab = take(sizeof(float) * rows * 2);
    p->off_vpart = take(sizeof(float) * rows * kHeadDim);
  }
  p->bwd_bytes = off;
  return RELPOS_OK;
}

bool ws_ok(const void* ws, size_t have, size_t need) {
  if (need == 0) return true;
  return ws != nullptr && have >= need && ((uintptr_t)ws % kAlign) == 0;
}

// Fills the per-call tables every pass needs (index maps, LUTs, row dots).
hipError_t run_prep(const relpos_desc* d, const Plan& p, const void* q, const void* k,
                    const void* rel_a, const void* rel_b, const float* bias_a, const float* bias_b,
                    char* ws, hipStream_t st) {
  const int L = p.L;
  const int64_t rows = (int64_t)p.B * p.H * L;
  hipError_t e = hipSuccess;
  if (d->mech == RELPOS_T5) {
    e = launch_index_map(MECH_T5, L, 0, 0, 0, p.t5, (int32_t*)(ws + p.off_bucket), nullptr, st);
    if (e != hipSuccess) return e;
    e = launch_t5_lut(bias_a, p.H, L, d->num_buckets, 1.0f / p.scale, p.t5, (float*)(ws + p.off_lut), st);
  } else if (d->mech == RELPOS_ALIBI) {
    // distinct "bucket" per offset and sign: no tile is single-valued, every tile adds the LUT
    e = launch_index_map(MECH_ALIBI, L, 0, 0, 0, p.t5, (int32_t*)(ws + p.off_bucket), nullptr, st);
    if (e != hipSuccess) return e;
    e = launch_alibi_lut(bias_a, p.H, L, 1.0f / p.scale, (float*)(ws + p.off_lut), st);
  } else if (d->mech == RELPOS_SHAW) {
    // end A (j - i >= k) reads w[2k], end B (j - i <= -k) reads w[0]
    RowDotArgs r{q, rows, L, p.H, rel_a, p.rel_hs, 2 * d->rel_span, 0, 2,
                 (float*)(ws + p.off_rowc), -1};
    e = launch_rowdot(r, p.fp32, p.fp32, st);
  } else if (d->mech == RELPOS_DEBERTA) {
    RowDotArgs r{q, rows, L, p.H, rel_a, p.rel_hs, 0, 2 * d->rel_span - 1, 2,
                 (float*)(ws + p.off_rowc), -1};
    e = launch_rowdot(r, p.fp32, p.fp32, st);
    if (e != hipSuccess) return e;
    RowDotArgs r2{k, rows, L, p.H, rel_b, p.rel_hs, 0, 2 * d->rel_span - 1, 2,
                  (float*)(ws + p.off_keyc), -1};
    e = launch_rowdot(r2, p.fp32, p.fp32, st);
  } else if (d->mech == RELPOS_TXL) {
    RowDotArgs r{k, rows, L, p.H, bias_a, kHeadDim, 0, 0, 1, (float*)(ws + p.off_uk), -1};
    e = launch_rowdot(r, p.fp32, true, st);
    if (e != hipSuccess) return e;
    // v_h . r_h[row] for every head and row (r_h = r + h rel_hs; the same table when shared)
    RowDotArgs r2{rel_a, (int64_t)p.H * p.nrel, p.nrel, p.H, bias_b, kHeadDim, 0, 0, 1,
                  (float*)(ws + p.off_vr), p.rel_hs};
    e = launch_rowdot(r2, p.fp32, true, st);
  }
  return e;
}

AttnShape make_shape(const relpos_desc* d, const Plan& p) {
  AttnShape s;
  s.B = p.B;
  s.H = p.H;
  s.L = p.L;
  s.wl = d->window_left;
  s.wr = d->window_right;
  s.mech = d->mech;   // RELPOS_* and MECH_* share their values
  s.span = d->rel_span;
  s.nrel = p.nrel;
  s.txl_off = p.txl_off;
  s.scale = p.scale;
  s.rel_hs = p.rel_hs;
  s.nbk = d->mech == RELPOS_T5 ? d->num_buckets : 0;
  s.t5sat = 1 << 30;
  s.t5b_pos = s.t5b_neg = 0;
  if (d->mech == RELPOS_T5) {
    // magnitudes at or past the last threshold share a side's last bucket (the unidirectional
    // map sends every delta <= 0 to bucket 0)
    const T5Map& m = p.t5;
    s.t5sat = m.nthr > 0 ? m.thr[m.nthr - 1] : m.max_exact;
    s.t5b_pos = m.max_exact + m.nthr;
    s.t5b_neg = m.bidirectional ? m.half + m.max_exact + m.nthr : 0;
  }
  return s;
}

// Table pointers each mechanism requires / forbids.
int check_tables(const relpos_desc* d, const void* rel_a, const void* rel_b, const void* bias_a,
                 const void* bias_b) {
  bool need_ra = false, need_rb = false, need_ba = false, need_bb = false;
  switch (d->mech) {
    case RELPOS_T5: need_ba = true; break;
    case RELPOS_ALIBI: need_ba = true; break;
    case RELPOS_SHAW: need_ra = true; break;
    case RELPOS_TXL: need_ra = need_ba = need_bb = true; break;
    case RELPOS_DEBERTA: need_ra = need_rb = true; break;
  }
  if ((rel_a != nullptr) != need_ra || (rel_b != nullptr) != need_rb) return RELPOS_E_INVALID;
  if ((bias_a != nullptr) != need_ba || (bias_b != nullptr) != need_bb) return RELPOS_E_INVALID;
  for (const void* ptr : {rel_a, rel_b, bias_a, bias_b})
    if (ptr && !aligned16(ptr)) return RELPOS_E_INVALID;
  return RELPOS_OK;
}

// profiling hook (see relpos_profile_events): per host thread, so that calls made from other
// threads never record the caller's events
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;
thread_local int g_prof_kernel = RELPOS_PROF_OFF;

template <typename F>
hipError_t timed(int which, hipStream_t st, F launch) {
  const bool on = g_prof_kernel == which;
  if (on) {
    hipError_t e = hipEventRecord(g_prof_start, st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (on && e == hipSuccess) e = hipEventRecord(g_prof_stop, st);
  return e;
}

// ------------------------------------------------------------------ projections
struct ProjPlan {
  bool fp32;
  int N, F, H, d, kslices;
  size_t ws_bytes;
};

int make_proj_plan(const relpos_proj_desc* d, ProjPlan* p) {
  if (!d) return RELPOS_E_INVALID;
  if (d->dtype != RELPOS_BF16 && d->dtype != RELPOS_FP32) return RELPOS_E_INVALID;
  if (d->rows < 0 || d->rows > (1 << 24)) return RELPOS_E_INVALID;
  if (d->in_features < 8 || d->in_features > 65536 || d->in_features % 8) return RELPOS_E_INVALID;
  if (d->heads < 1 || d->head_dim < 8 || d->head_dim % 8) return RELPOS_E_INVALID;
  if (d->heads * d->head_dim > 65536) return RELPOS_E_INVALID;
  p->fp32 = d->dtype == RELPOS_FP32;
  p->N = (int)d->rows;
  p->F = (int)d->in_features;
  p->H = (int)d->heads;
  p->d = (int)d->head_dim;
  // about one 128 x 128 dW tile-slice per compute unit, each slice at least one 64-row k step
  const int tiles = ((p->F + 127) / 128) * ((p->H * p->d + 127) / 128);
  p->kslices = std::max(1, std::min(256 / tiles, (p->N + 63) / 64));
  p->ws_bytes = p->kslices > 1
                    ? align_up((size_t)p->kslices * p->F * p->H * p->d * sizeof(float)) : 0;
  return RELPOS_OK;
}

}  // namespace

extern "C" {

int relpos_profile_events(hipEvent_t start_event, hipEvent_t stop_event, int kernel) {
  if (kernel == RELPOS_PROF_OFF) {
    g_prof_kernel = RELPOS_PROF_OFF;
    g_prof_start = g_prof_stop = nullptr;
    return RELPOS_OK;
  }
  if (kernel < RELPOS_PROF_FWD || kernel > RELPOS_PROF_BWD_DKDV || !start_event || !stop_event)
    return RELPOS_E_INVALID;
  g_prof_start = start_event;
  g_prof_stop = stop_event;
  g_prof_kernel = kernel;
  return RELPOS_OK;
}

int relpos_version(void) { return 200; }

const char* relpos_status_string(int status) {
  switch (status) {
    case RELPOS_OK: return "ok";
    case RELPOS_E_INVALID: return "invalid argument";
    case RELPOS_E_UNSUPPORTED: return "unsupported configuration";
    case RELPOS_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case RELPOS_E_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int relpos_attn_workspace_size(const relpos_desc* desc, int pass, size_t* bytes) {
  if (!bytes || (pass != 0 && pass != 1)) return RELPOS_E_INVALID;
  Plan p;
  int st = make_plan(desc, &p);
  if (st != RELPOS_OK) return st;
  *bytes = pass == 0 ? p.fwd_bytes : p.bwd_bytes;
  return RELPOS_OK;
}

int relpos_index_map(const relpos_desc* desc, int32_t* out_a, int32_t* out_b, hipStream_t stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != RELPOS_OK) return st;
  if (p.L == 0) return RELPOS_OK;
  if (!out_a || !aligned16(out_a)) return RELPOS_E_INVALID;
  if ((desc->mech == RELPOS_DEBERTA) != (out_b != nullptr)) return RELPOS_E_INVALID;
  if (out_b && !aligned16(out_b)) return RELPOS_E_INVALID;
  hipError_t e = launch_index_map(desc->mech == RELPOS_ALIBI ? MECH_ALIBI : desc->mech, p.L, desc->rel_span, p.nrel, p.txl_off, p.t5, out_a,
                                  out_b, stream);
  return e == hipSuccess ? RELPOS_OK : RELPOS_E_LAUNCH;
}

int relpos_attn_fwd(const relpos_desc* desc, const void* q, const void* k, const void* v,
                    const void* rel_a, const void* rel_b, const float* bias_a, const float* bias_b,
                    void* o, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != RELPOS_OK) return st;
  st = check_tables(desc, rel_a, rel_b, bias_a, bias_b);
  if (st != RELPOS_OK) return st;
  if (p.B == 0 || p.L == 0) return RELPOS_OK;
  for (const void* ptr : {q, k, v, (const void*)o, (const void*)lse})
    if (!ptr || !aligned16(ptr)) return RELPOS_E_INVALID;
  if (!ws_ok(workspace, workspace_bytes, p.fwd_bytes)) return RELPOS_E_WORKSPACE;
  hipStream_t s = stream;
  char* ws = (char*)workspace;
  hipError_t e = run_prep(desc, p, q, k, rel_a, rel_b, bias_a, bias_b, ws, s);
  if (e != hipSuccess) return RELPOS_E_LAUNCH;
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.sh = make_shape(desc, p);
  a.q = q; a.k = k; a.v = v;
  a.rel_a = rel_a; a.rel_b = rel_b;
  a.o = o; a.lse = lse;
  if (desc->mech == RELPOS_T5 || desc->mech == RELPOS_ALIBI) {
    a.lut = (const float*)(ws + p.off_lut);
    a.bucket = (const int*)(ws + p.off_bucket);
  }
  if (desc->mech == RELPOS_ALIBI) a.slopes = bias_a;
  if (desc->mech == RELPOS_SHAW || desc->mech == RELPOS_DEBERTA) a.rowc = (const float*)(ws + p.off_rowc);
  if (desc->mech == RELPOS_DEBERTA) a.keyc = (const float*)(ws + p.off_keyc);
  if (desc->mech == RELPOS_TXL) {
    a.uk = (const float*)(ws + p.off_uk);
    a.vr = (const float*)(ws + p.off_vr);
  }
  e = timed(RELPOS_PROF_FWD, s, [&] { return launch_fwd(a, p.fp32, s); });
  return e == hipSuccess ? RELPOS_OK : RELPOS_E_LAUNCH;
}

int relpos_attn_bwd(const relpos_desc* desc, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dout, const void* rel_a,
                    const void* rel_b, const float* bias_a, const float* bias_b, void* dq, void* dk,
                    void* dv, float* drel_a, float* drel_b, float* dbias_a, float* dbias_b,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != RELPOS_OK) return st;
  st = check_tables(desc, rel_a, rel_b, bias_a, bias_b);
  if (st != RELPOS_OK) return st;
  // every table has its gradient slot, and no other slot is set
  if ((drel_a != nullptr) != (rel_a != nullptr) || (drel_b != nullptr) != (rel_b != nullptr) ||
      (dbias_a != nullptr) != (bias_a != nullptr) || (dbias_b != nullptr) != (bias_b != nullptr))
    return RELPOS_E_INVALID;
  for (const void* ptr : {(const void*)drel_a, (const void*)drel_b, (const void*)dbias_a, (const void*)dbias_b})
    if (ptr && !aligned16(ptr)) return RELPOS_E_INVALID;
  hipStream_t s = stream;
  if (p.B == 0 || p.L == 0) {
    // no pairs: every table gradient is zero (nrel is clamped at 0 when L = 0)
    size_t n_a = 0, n_b = 0, n_ba = 0, n_bb = 0;
    const size_t H = (size_t)p.H;
    const size_t tabs = p.rel_hs ? H : 1;   // per-head relation tables or one shared table
    const size_t rel = tabs * (size_t)p.rel_rows * kHeadDim;
    switch (desc->mech) {
      case RELPOS_T5: n_ba = H * desc->num_buckets; break;
      case RELPOS_ALIBI: n_ba = H; break;
      case RELPOS_SHAW: n_a = rel; break;
      case RELPOS_TXL: n_a = rel; n_ba = n_bb = H * kHeadDim; break;
      case RELPOS_DEBERTA: n_a = n_b = rel; break;
    }
    hipError_t e = hipSuccess;
    if (n_a) e = launch_agg_rows(nullptr, 0, 0, (int64_t)n_a, 0.f, drel_a, s);
    if (e == hipSuccess && n_b) e = launch_agg_rows(nullptr, 0, 0, (int64_t)n_b, 0.f, drel_b, s);
    if (e == hipSuccess && n_ba) e = launch_agg_rows(nullptr, 0, 0, (int64_t)n_ba, 0.f, dbias_a, s);
    if (e == hipSuccess && n_bb) e = launch_agg_rows(nullptr, 0, 0, (int64_t)n_bb, 0.f, dbias_b, s);
    return e == hipSuccess ? RELPOS_OK : RELPOS_E_LAUNCH;
  }
  for (const void* ptr : {q, k, v, o, (const void*)lse, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!ptr || !aligned16(ptr)) return RELPOS_E_INVALID;
  if (!ws_ok(workspace, workspace_bytes, p.bwd_bytes)) return RELPOS_E_WORKSPACE;
  char* ws = (char*)workspace;
  hipError_t e = run_prep(desc, p, q, k, rel_a, rel_b, bias_a, bias_b, ws, s);
  if (e != hipSuccess) return RELPOS_E_LAUNCH;
  const int64_t rows = (int64_t)p.B * p.H * p.L;
  e = launch_dsum(o, dout, rows, p.fp32, (float*)(ws + p.off_dsum), s);
  if (e != hipSuccess) return RELPOS_E_LAUNCH;

  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.sh = make_shape(desc, p);
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.lse = lse;
  a.dsum = (const float*)(ws + p.off_dsum);
  a.rel_a = rel_a; a.rel_b = rel_b;
  a.bias_a = bias_a; a.bias_b = bias_b;
  a.fold = p.fold;
  a.fold_slices = p.fold_slices ? 1 : 0;
  if (desc->mech == RELPOS_T5 || desc->mech == RELPOS_ALIBI) {
    a.lut = (const float*)(ws + p.off_lut);
    a.bucket = (const int*)(ws + p.off_bucket);
  }
  if (desc->mech == RELPOS_SHAW || desc->mech == RELPOS_DEBERTA) a.rowc = (const float*)(ws + p.off_rowc);
  if (desc->mech == RELPOS_DEBERTA) a.keyc = (const float*)(ws + p.off_keyc);
  if (desc->mech == RELPOS_TXL) {
    a.uk = (const float*)(ws + p.off_uk);
    a.vr = (const float*)(ws + p.off_vr);
  }
  a.dq = dq; a.dk = dk; a.dv = dv;
  if (p.part_q_stride) a.part_q = (float*)(ws + p.off_part_q);
  if (p.part_k_stride) a.part_k = (float*)(ws + p.off_part_k);
  if (p.off_part_qv) a.part_qv = (float*)(ws + p.off_part_qv);
  if (p.off_part_kv) a.part_kv = (float*)(ws + p.off_part_kv);
  a.part_q_stride = p.part_q_stride;
  a.part_k_stride = p.part_k_stride;
  if (p.off_xpart) a.xpart = (float*)(ws + p.off_xpart);
  if (p.off_vpart) a.vpart = (float*)(ws + p.off_vpart);
  if (p.off_cab) a.cab = (float*)(ws + p.off_cab);

  e = timed(RELPOS_PROF_BWD_DQ, s, [&] { return launch_bwd_dq(a, p.fp32, s); });
  if (e != hipSuccess) return RELPOS_E_LAUNCH;
  const bool rev = desc->window_right == 0;
  float* diag = p.off_diag ? (float*)(ws + p.off_diag) : nullptr;
  if (desc->mech == RELPOS_TXL) {
    // the per-offset sums of the query-side pass, then the key-side pass and its r partials
    e = launch_agg_diag(a.part_qv, p.B, p.H, p.L, p.nb, rev, desc->window_left, desc->window_right, diag, s);
    if (p.txl_group == 0) {
      // batch entries folded: `fold` launches over ceil(B / fold) H slices' workgroups, each
      // adding to the partials of the one before, then one aggregation
      const int ng = (p.B + p.fold - 1) / p.fold;
      a.bh0 = 0;
      a.nbh = ng * p.H;
      e = timed(RELPOS_PROF_BWD_DKDV, s, [&] {
        hipError_t r = hipSuccess;
        for (a.sub = 0; a.sub < p.fold && r == hipSuccess; ++a.sub) r = launch_bwd_dkdv(a, p.fp32, s);
        return r;
      });
      if (e == hipSuccess)
        e = launch_agg_txl_dr(a.part_q, diag, bias_b, p.H, p.L, p.nb,
                              (int)(p.part_q_stride / kHeadDim), desc->window_left,
                              desc->window_right, p.nrel, p.txl_off, p.scale, 0, ng * p.H,
                              ng * p.H, true, true, p.rel_hs == 0, drel_a, s);
    }
    const int nbh = p.B * p.H, G = p.txl_group;
    if (G > 0 && e == hipSuccess) {
      // slice groups, each group's r partials folded into dr before the next reuses them
      e = timed(RELPOS_PROF_BWD_DKDV, s, [&] {
        hipError_t r = hipSuccess;
        for (int s0 = 0; s0 < nbh && r == hipSuccess; s0 += G) {
          a.bh0 = s0;
          a.nbh = std::min(G, nbh - s0);
          r = launch_bwd_dkdv(a, p.fp32, s);
          if (r == hipSuccess)
            r = launch_agg_txl_dr(a.part_q, diag, bias_b, p.H, p.L, p.nb,
                                  (int)(p.part_q_stride / kHeadDim), desc->window_left,
                                  desc->window_right, p.nrel, p.txl_off, p.scale, s0, a.nbh,
                                  nbh, s0 == 0, s0 + G >= nbh, p.rel_hs == 0, drel_a, s);
        }
        return r;
      });
    }
    if (e == hipSuccess)
      e = launch_agg_txl_uv(a.part_kv, diag, rel_a, p.rel_hs, p.B, p.H, p.L, p.nb, p.nrel,
                            p.txl_off, p.scale, p.fp32, dbias_a, dbias_b, s);
    return e == hipSuccess ? RELPOS_OK : RELPOS_E_LAUNCH;
  }
  e = timed(RELPOS_PROF_BWD_DKDV, s, [&] { return launch_bwd_dkdv(a, p.fp32, s); });
  if (e != hipSuccess) return RELPOS_E_LAUNCH;

  switch (desc->mech) {
    case RELPOS_T5:
      // dbeta[h][k]: the bucket sums of head h's owners, in ascending (batch, block) order
      e = launch_agg_rows_by_head(a.part_qv, desc->num_buckets, p.B, p.H, p.nb, desc->num_buckets,
                                  1.0f, dbias_a, s);
      break;
    case RELPOS_ALIBI:
      e = launch_agg_alibi(a.part_qv, p.B, p.H, p.nb, dbias_a, s);
      break;
    case RELPOS_SHAW:
    case RELPOS_DEBERTA: {
      // one shared table sums every slot (slot g nb + p for slice group g); per-head tables
      // sum the slots of their head (slot (g H + h) nb + p for batch group g)
      auto agg = [&](const float* part, int64_t stride, float* out) {
        const int ng = (p.B + p.fold - 1) / p.fold;
        return p.rel_hs == 0
                   ? launch_agg_rows(part, stride, p.fold_owners, stride, p.scale, out, s)
                   : launch_agg_rows_by_head(part, stride, ng, p.H, p.nb, stride, p.scale, out, s);
      };
      e = agg(a.part_q, p.part_q_stride, drel_a);
      if (e == hipSuccess && desc->mech == RELPOS_DEBERTA) e = agg(a.part_k, p.part_k_stride, drel_b);
      break;
    }
    default:
      break;
  }
  return e == hipSuccess ? RELPOS_OK : RELPOS_E_LAUNCH;
}

int relpos_project_fwd(const relpos_proj_desc* desc, const void* X, const void* W, void* rel,
                       hipStream_t stream) {
  ProjPlan p;
  int st = make_proj_plan(desc, &p);
  if (st != RELPOS_OK) return st;
  if (p.N == 0) return RELPOS_OK;
  for (const void* ptr : {X, W, (const void*)rel})
    if (!ptr || !aligned16(ptr)) return RELPOS_E_INVALID;
  hipError_t e = launch_project_fwd(X, W, rel, p.N, p.F, p.H, p.d, p.fp32, stream);
  return e == hipSuccess ? RELPOS_OK : RELPOS_E_LAUNCH;
}

int relpos_project_workspace_size(const relpos_proj_desc* desc, size_t* bytes) {
  if (!bytes) return RELPOS_E_INVALID;
  ProjPlan p;
  int st = make_proj_plan(desc, &p);
  if (st != RELPOS_OK) return st;
  *bytes = p.ws_bytes;
  return RELPOS_OK;
}

int relpos_project_bwd(const relpos_proj_desc* desc, const void* X, const void* W,
                       const float* drel, float* dX, float* dW, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  ProjPlan p;
  int st = make_proj_plan(desc, &p);
  if (st != RELPOS_OK) return st;
  if (!dX && !dW) return RELPOS_OK;
  for (const void* ptr : {X, W, (const void*)drel})
    if (p.N > 0 && (!ptr || !aligned16(ptr))) return RELPOS_E_INVALID;
  if (dX && !aligned16(dX)) return RELPOS_E_INVALID;
  if (dW && !aligned16(dW)) return RELPOS_E_INVALID;
  if (dW && !X) return RELPOS_E_INVALID;
  if (dW && p.ws_bytes && !ws_ok(workspace, workspace_bytes, p.ws_bytes))
    return RELPOS_E_WORKSPACE;
  hipError_t e = launch_project_bwd(X, W, drel, dX, dW, (float*)workspace, p.kslices, p.N, p.F,
                                    p.H, p.d, p.fp32, stream);
  return e == hipSuccess ? RELPOS_OK : RELPOS_E_LAUNCH;
}

}  // extern "C"
