// Forward kernel: exact softmax attention with additive relative-position terms, one
// workgroup per (batch, head, 128-query block), keys streamed in 64-row tiles with an
// online softmax.  The relative term is folded into the score tile and never stored (abstract
// of "Fast and Exact Relative-Position Attention via Structure-Aware Kernels"; zicq.com
// explainer, section on how structure-aware tiling stays exact: B is added inside the online
// softmax accumulation instead of being built as a full matrix first).
//
// Scores are kept in "y units": y = q.k + (relative term) / s, the natural logit being s*y.
// exp(s*y - s*m) = exp2(y * c - m * c) with c = s * log2(e).
#include "relpos_tile.h"

namespace relpos {

template <typename T, int MECH>
__device__ __forceinline__ void fwd_body(const FwdArgs& a) {
  constexpr int NP = Elem<T>::NP;
  constexpr bool LUTP = (MECH == MECH_T5 || MECH == MECH_ALIBI);   // per-offset bias LUT path
  constexpr bool REL = !LUTP;
  constexpr bool VEC = LUTP;
  constexpr int KVEC = (MECH == MECH_DEBERTA || MECH == MECH_ALIBI) ? 2 * BOTH
                                                                    : (MECH == MECH_TXL ? BOTH : 1);
  __shared__ __attribute__((aligned(16))) uint16_t ks[NP * BOTH * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vs[NP * BOTH * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t win[REL ? NP * WIN * TSTR : 8];
  __shared__ __attribute__((aligned(16))) float gsb[REL ? NWAVE * WROWS * GS2 : 4];
  __shared__ __attribute__((aligned(16))) float vec_s[VEC ? WIN : 4];   // T5 LUT slice
  // T-XL u.k / DeBERTa k.Qr ends / ALiBi ramps +m y / s and -m y / s over a key tile
  __shared__ __attribute__((aligned(16))) float kvec_s[KVEC];

  const AttnShape sh = a.sh;
  const int L = sh.L;
  const int nqb = (L + BLANE - 1) / BLANE;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int qb = bid % nqb;
  const int bh = bid / nqb;
  if (sh.wr == 0) qb = nqb - 1 - qb;   // causal: longest rows first
  const int h = bh % sh.H;
  const int i0 = qb * BLANE;

  const int tid = threadIdx.x;
  const int w = wave_index();
  const int lane = tid & 63;
  const int l32 = lane & 31, kh = lane >> 5;
  const int qw0 = i0 + WROWS * w;
  const int my_i = qw0 + l32;
  const bool lane_valid = my_i < L;   // rows past L are padding (no allowed key)

  const int64_t bh_off = (int64_t)bh * L * kHeadDim;
  const T* qg = (const T*)a.q + bh_off;
  const T* kg = (const T*)a.k + bh_off;
  const T* vg = (const T*)a.v + bh_off;
  const float s = sh.scale;
  const float c = s * kLog2e;
  const int span = sh.span;

  // Lane-side operand: this lane's query row.
  Op<NP> qop[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    if (my_i < L) {
      qop[cc] = op_from_global<T>(qg + (int64_t)my_i * kHeadDim + 16 * cc + 8 * kh);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      qop[cc] = op_from_f32<NP>(z);
    }
  }
  // Clipped-end constants of this query row: the products with the table row shared by all
  // offsets delta <= -k (end A) and by all large offsets (end B).  Shaw: A = w[2k], B = w[0];
  // DeBERTa: A = Kr[0], B = Kr[2k-1].
  float rcA = 0.f, rcB = 0.f;
  if constexpr (MECH == MECH_SHAW || MECH == MECH_DEBERTA) {
    if (my_i < L) {
      rcA = a.rowc[((int64_t)bh * L + my_i) * 2 + 0];
      rcB = a.rowc[((int64_t)bh * L + my_i) * 2 + 1];
    }
  }

  // ALiBi: on a wave tile on one side of the diagonal, -m |i - j| / s = (row term) + (key
  // term) with the key term a ramp over the tile's 64 keys: the ramp starts the score
  // accumulators and the row term joins the row constant, so those tiles add nothing per
  // element.  Tiles that straddle the diagonal read the per-offset LUT.
  float am = 0.f;   // ALiBi: m / s
  if constexpr (MECH == MECH_ALIBI) {
    am = a.slopes[h] / s;
    if (tid < BOTH) {
      kvec_s[tid] = am * (float)tid;
      kvec_s[BOTH + tid] = -am * (float)tid;
    }
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[2] = {f32x16{}, f32x16{}};

  // Key range of this workgroup under the mask.
  int j_lo = 0, j_hi = L - 1;
  if (sh.wl >= 0) j_lo = max(0, i0 - sh.wl);
  if (sh.wr >= 0) j_hi = min(L - 1, i0 + BLANE - 1 + sh.wr);
  const int jt0 = (j_lo / BOTH) * BOTH;

  float* gs = gsb + (REL ? w * WROWS * GS2 : 0);

  // K and V of the next tile are read into registers while the current tile computes
  TilePrefetch<T> pk, pv;
  if (jt0 <= j_hi) {
    pk.load(kg, jt0, L);
    pv.load(vg, jt0, L);
  }
  // T-XL: the window slides by 64 offsets per key tile, so it is kept circular (rotation
  // xrot) and only the 64 new table rows, their v.r values and the next keys' u.k are read
  // per tile, into registers one tile ahead
  TilePrefetch<T> pw;
  float pvr = 0.f, puk = 0.f;
  // T5 / ALiBi: this thread's LUT entry of the next tile's window (window row x = tid)
  float plut = 0.f;
  auto lut_load = [&](int j0x) {
    if (tid < WIN) {
      const int d = i0 - (j0x + BOTH - 1) + tid;
      plut = (d > -L && d < L) ? a.lut[(int64_t)h * (2 * L - 1) + d + L - 1] : 0.f;
    }
  };
  if constexpr (LUTP) {
    if (jt0 <= j_hi) lut_load(jt0);
  }
  // DeBERTa: end A / end B constants of the next tile's keys (threads 0..127)
  float pkc = 0.f;
  auto kc_load = [&](int j0x) {
    if (tid < 2 * BOTH) {
      const int jj = j0x + (tid >> 1);
      pkc = (jj < L) ? a.keyc[((int64_t)bh * L + jj) * 2 + (tid & 1)] : 0.f;
    }
  };
  if constexpr (MECH == MECH_DEBERTA) {
    if (jt0 <= j_hi) kc_load(jt0);
  }
  const T* rtab = nullptr;
  if constexpr (MECH == MECH_TXL) rtab = (const T*)a.rel_a + h * sh.rel_hs;
  if constexpr (MECH == MECH_TXL) {
    // The first key tile's window (192 table rows and their v.r values) and u.k, staged before
    // the sweep (the first barrier inside the loop orders these writes before any read).  Taken
    // inside the loop on the first step only, these reads would sit in branches the compiler
    // cannot rule out on later steps, and it would wait for every read in flight (the next
    // tile's prefetch included) before reusing their registers.
    if (jt0 <= j_hi) {
      const int dlo0 = i0 - (jt0 + BOTH - 1), nrel = sh.nrel, toff = sh.txl_off;
      stage_window<T, NP>(win, rtab, [&](int x) { return row_side_row(MECH, dlo0 + x, span, nrel, toff); });
      for (int x = tid; x < WIN; x += 256) {
        const int r = row_side_row(MECH, dlo0 + x, span, nrel, toff);
        *win_vec(win, x) = (r >= 0) ? a.vr[(int64_t)h * nrel + r] : 0.f;
      }
      if (tid < BOTH) kvec_s[tid] = (jt0 + tid < L) ? a.uk[(int64_t)bh * L + jt0 + tid] : 0.f;
    }
  }

  for (int j0 = jt0; j0 <= j_hi; j0 += BOTH) {
    // circular T-XL window: row x of step s sits at physical row (x - 64 s) mod 192
    const int xrot = (MECH == MECH_TXL) ? ((3 - ((j0 - jt0) / BOTH) % 3) % 3) * BOTH : 0;
    // ---- tile classification (offset-aware scheduling) ----
    // wave tile offsets delta = i - j in [dlo, dhi]
    const int dlo = qw0 - (j0 + BOTH - 1), dhi = qw0 + WROWS - 1 - j0;
    const int wg_dlo = i0 - (j0 + BOTH - 1), wg_dhi = i0 + BLANE - 1 - j0;
    const int dlo_c = clampi(dlo, 1 - L, L - 1), dhi_c = clampi(dhi, 1 - L, L - 1);
    bool wave_none = (j0 >= L) || (qw0 >= L);
    if (sh.wl >= 0 && dlo > sh.wl) wave_none = true;
    if (sh.wr >= 0 && -dhi > sh.wr) wave_none = true;
    bool wave_full = (j0 + BOTH <= L) && (sh.wl < 0 || dhi <= sh.wl) && (sh.wr < 0 || -dlo <= sh.wr);
    // relative-term class: 0 general, 1 clipped low (delta small), 2 clipped high
    int cls = 0;
    bool wg_general = true;
    if constexpr (MECH == MECH_SHAW) {
      // row = clamp(j - i, -k, k) + k: clipped when j - i >= k (hi row) or <= -k (row 0)
      if (-dhi >= span) cls = 2; else if (-dlo <= -span) cls = 1;
      wg_general = !((-wg_dhi >= span) || (-wg_dlo <= -span));
    } else if constexpr (MECH == MECH_DEBERTA) {
      if (dlo >= span) cls = 2; else if (dhi <= -span) cls = 1;
      wg_general = !((wg_dlo >= span) || (wg_dhi <= -span));
    } else if constexpr (MECH == MECH_ALIBI) {
      // side of the diagonal: 1 every i >= j, 2 every i < j, 0 both
      if (dlo >= 0) cls = 1; else if (dhi < 0) cls = 2;
    } else if constexpr (MECH == MECH_T5) {
      // one bucket for the whole wave tile: the offsets lie on one side of 0 (where the
      // bucket map is monotone) and both ends share a bucket; past the last threshold on
      // either side without reading the map
      if (dlo_c >= sh.t5sat || dhi_c <= -sh.t5sat)
        cls = 1;
      else if ((dlo_c >= 0 || dhi_c < 0) && a.bucket[dlo_c + L - 1] == a.bucket[dhi_c + L - 1])
        cls = 1;
    }

    __syncthreads();  // previous tile's LDS reads are done
    pk.store(ks);
    pv.store(vs);
    if constexpr (LUTP) {
      // (ALiBi reads the slice only on workgroup tiles that straddle the diagonal)
      if ((MECH != MECH_ALIBI || (wg_dlo < 0 && wg_dhi >= 0)) && tid < WIN) vec_s[tid] = plut;
      if (j0 + BOTH <= j_hi) lut_load(j0 + BOTH);
    } else if constexpr (MECH == MECH_TXL) {
      if (j0 != jt0) {
        // window rows 0..63 are new: physical rows xrot .. xrot + 63 (the rows that left)
        pw.store_at(win, WIN * TSTR, xrot);
        if (tid < BOTH) {
          *win_vec(win, xrot + tid) = pvr;
          kvec_s[tid] = puk;
        }
      }
    } else if (wg_general) {
      const int toff = sh.txl_off, nrel = sh.nrel;
      const T* tab = (const T*)a.rel_a + h * sh.rel_hs;
      stage_window<T, NP>(win, tab, [&](int x) {
        return row_side_row(MECH, wg_dlo + x, span, nrel, toff);
      });
    }
    if constexpr (MECH == MECH_DEBERTA) {
      // end A values of the 64 keys, then end B: each a contiguous vector
      if (tid < 2 * BOTH) kvec_s[(tid & 1) * BOTH + (tid >> 1)] = pkc;
    }
    if (j0 + BOTH <= j_hi) {
      pk.load(kg, j0 + BOTH, L);
      pv.load(vg, j0 + BOTH, L);
      if constexpr (MECH == MECH_DEBERTA) kc_load(j0 + BOTH);
      if constexpr (MECH == MECH_TXL) {
        // next tile's new window rows: offsets wg_dlo - 64 .. wg_dlo - 1
        const int r0 = wg_dlo - BOTH + sh.txl_off;
        pw.load_range(rtab, r0, 0, sh.nrel);
        pvr = 0.f;
        puk = 0.f;
        if (tid < BOTH) {
          if (r0 + tid >= 0 && r0 + tid < sh.nrel) pvr = a.vr[(int64_t)h * sh.nrel + r0 + tid];
          if (j0 + BOTH + tid < L) puk = a.uk[(int64_t)bh * L + j0 + BOTH + tid];
        }
      }
    }
    __syncthreads();

    f32x16 sc[2];
    Op<NP> kop[2][4];
    if (!wave_none) {
      if constexpr (MECH == MECH_TXL) {
        // T-XL: the scores start from u.k of each key
        other_dot_lane<NP, true>(sc, ks, qop, kop, kvec_s);
      } else if constexpr (MECH == MECH_DEBERTA) {
        // a clipped wave tile starts its scores from the keys' end-row constants
        if (cls != 0) other_dot_lane<NP, true>(sc, ks, qop, kop, kvec_s + (cls == 2 ? 0 : BOTH));
        else other_dot_lane<NP>(sc, ks, qop, kop);
      } else if constexpr (MECH == MECH_ALIBI) {
        // i >= j: -m (i - j0) / s + m (j - j0) / s; i < j: m (i - j0) / s - m (j - j0) / s
        if (cls != 0) other_dot_lane<NP, true>(sc, ks, qop, kop, kvec_s + (cls == 1 ? 0 : BOTH));
        else other_dot_lane_offset<NP>(sc, ks, qop, kop, vec_s, WROWS * w);
      } else if constexpr (MECH == MECH_T5) {
        // a one-bucket wave tile adds its bias as a row constant; others start the
        // accumulators from the per-offset bias
        if (cls == 1) other_dot_lane<NP>(sc, ks, qop, kop);
        else other_dot_lane_offset<NP>(sc, ks, qop, kop, vec_s, WROWS * w);
      } else {
        other_dot_lane<NP>(sc, ks, qop, kop);
      }
    }
    float rowconst = 0.f;
    // ---- relative terms (row side) ----
    if constexpr (MECH == MECH_T5) {
      if (!wave_none && cls == 1) rowconst = vec_s[dlo_c - wg_dlo];
    } else if constexpr (MECH == MECH_ALIBI) {
      if (!wave_none) {
        if (cls == 1) rowconst = -am * (float)(my_i - j0);
        else if (cls == 2) rowconst = am * (float)(my_i - j0);
      }
    } else if constexpr (MECH == MECH_SHAW) {
      if (!wave_none) {
        if (cls == 2) rowconst = rcA;        // j - i >= k: row 2k
        else if (cls == 1) rowconst = rcB;   // j - i <= -k: row 0
        else {
          f32x16 g[3];
          row_products<NP, false>(g, win, WROWS * w, qop);
          row_skew_add(sc, g, gs);
        }
      }
    } else if constexpr (MECH == MECH_TXL) {
      if (!wave_none) {
        f32x16 g[3];
        row_products<NP, true, true>(g, win, WROWS * w, qop, xrot);
        row_skew_add(sc, g, gs);
      }
    } else if constexpr (MECH == MECH_DEBERTA) {
      if (!wave_none) {
        if (cls == 2) rowconst = rcB;        // delta >= k (key term in the accumulator start)
        else if (cls == 1) rowconst = rcA;   // delta <= -k
        else {
          f32x16 g[3];
          row_products<NP, false>(g, win, WROWS * w, qop);
          row_skew_add(sc, g, gs);
        }
      }
      if (wg_general) {
        // column side (p2c): restage the window with Qr rows
        __syncthreads();
        stage_window<T, NP>(win, (const T*)a.rel_b + h * sh.rel_hs, [&](int x) {
          // column window row x <-> rho = j - i = (j0 - i0 - 127) + x
          return p2c_row(-((j0 - i0 - (BLANE - 1)) + x), span);
        });
        __syncthreads();
        if (!wave_none && cls == 0) {
#pragma unroll
          for (int ob = 0; ob < 2; ++ob)
            col_skew_add<NP, false>(sc, win, (BLANE - WROWS) - WROWS * w, ob, ks, gs);
        }
      }
    }
    if (wave_none) continue;

    // ---- mask ----
    if (!wave_full) {
      const int wlx = sh.wl < 0 ? L : sh.wl, wrx = sh.wr < 0 ? L : sh.wr;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * b + 8 * (r >> 2) + 4 * kh + (r & 3);
          sc[b][r] = pair_ok(my_i, j, L, wlx, wrx) ? sc[b][r] : kNegInf;
        }
    }

    // ---- online softmax ----
    // The weights are formed against the row's running reference m_run (y units): a tile whose
    // scores stay below m_run + 12 / c keeps every weight below 2^12, and the sums and the O
    // accumulator stay exact in fp32 without a rescale, so neither the tile's row maximum nor a
    // rescale is needed.  Only when a row of the wave has no reference yet (its first allowed
    // keys) or a lane's weights sum past 2^12 (the scores grew; inf included) does the wave take
    // the exact path: row maxima, the rescale of O and l by exp2((m_old - m_new) c), and the
    // weights again.  The normalisation O = acc / l and LSE = s m_run + ln l are exact for any
    // reference, so both paths give the same softmax up to rounding.
    Op<NP> pop[4];
    float psum = 0.f;
    auto weights = [&](float m_ref) {
      const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
      const float bias = (rowconst - m_use) * c;
      float ps = 0.f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float x[8];
        const f32x16& v = sc[cc >> 1];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          x[i] = fast_exp2(fmaf(v[8 * (cc & 1) + i], c, bias));
          if constexpr (NP == 2) ps += x[i];
        }
        pop[cc] = op_from_f32<NP>(x);
      }
      // bf16: the denominator sums exactly the rounded weights that multiply V
      if constexpr (NP == 1) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) ps = sum_bf16x8(pop[cc].p[0], ps);
      }
      return ps;
    };
    // ALiBi's scores climb toward the diagonal by m per key, so most tiles before it would
    // cross the bound: it takes the exact path on every tile.
    bool exact = (MECH == MECH_ALIBI) || __any(lane_valid && m_run == kNegInf);
    if (!exact) {
      psum = weights(m_run);
      exact = __any(!(psum <= 4096.f));
    }
    if (exact) {
      float mx = kNegInf;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = max3f(mx, sc[b][r], sc[b][r + 1]);
      mx = max3f(mx, xhalf(mx), kNegInf);
      mx += rowconst;
      const bool raise = mx > m_run;
      const float m_new = raise ? mx : m_run;
      const float alpha = raise ? fast_exp2((m_run - m_new) * c) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db) oacc[db] *= alpha;
      m_run = m_new;
      psum = weights(m_run);
    }
    l_run += psum;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        Op<NP> vop = op_rows_tr<NP>(vs, BOTH * TSTR, TSTR, 16 * cc, 32 * db);
        mma<NP>(oacc[db], vop, pop[cc]);
      }
    }
  }

  // ---- epilogue ----
  const float l_tot = l_run + xhalf(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (my_i < L) {
    T* og = (T*)a.o + bh_off + (int64_t)my_i * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * kh;
        float o0 = oacc[db][4 * g] * inv, o1 = oacc[db][4 * g + 1] * inv;
        float o2 = oacc[db][4 * g + 2] * inv, o3 = oacc[db][4 * g + 3] * inv;
        if constexpr (NP == 1) {
          u32x2 pk = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          *(u32x2*)(og + d) = pk;
        } else {
          f32x4 v4 = {o0, o1, o2, o3};
          *(f32x4*)(og + d) = v4;
        }
      }
    if (kh == 0) {
      a.lse[(int64_t)bh * L + my_i] = (l_tot > 0.f) ? (s * m_run + logf(l_tot)) : kNegInf;
    }
  }
}

// Two workgroups (8 waves) per CU when the LDS footprint allows it (bf16); the launch bound
// caps registers at 256 per lane so the register file does not become the limit instead.
template <typename T, int MECH>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  fwd_body<T, MECH>(a);
}
template <typename T, int MECH>
__global__ __launch_bounds__(256, 1) void fwd_kernel_1wg(FwdArgs a) {
  fwd_body<T, MECH>(a);
}
// T5 and ALiBi keep only K, V and a LUT slice in LDS (19 KB): three workgroups per CU when
// the registers fit 168 per lane.
template <typename T, int MECH>
__global__ __launch_bounds__(256, 3) void fwd_kernel_3wg(FwdArgs a) {
  fwd_body<T, MECH>(a);
}

template <typename T, int MECH>
static void launch_one(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (Elem<T>::NP == 1 && (MECH == MECH_T5 || MECH == MECH_ALIBI))
    hipLaunchKernelGGL((fwd_kernel_3wg<T, MECH>), grid, dim3(256), 0, stream, a);
  else if constexpr (Elem<T>::NP == 1)
    hipLaunchKernelGGL((fwd_kernel<T, MECH>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_kernel_1wg<T, MECH>), grid, dim3(256), 0, stream, a);
}

template <typename T>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.sh.L + BLANE - 1) / BLANE;
  const dim3 grid((unsigned)(nqb * a.sh.B * a.sh.H));
  switch (a.sh.mech) {
    case MECH_T5: launch_one<T, MECH_T5>(a, grid, stream); break;
    case MECH_SHAW: launch_one<T, MECH_SHAW>(a, grid, stream); break;
    case MECH_TXL: launch_one<T, MECH_TXL>(a, grid, stream); break;
    case MECH_DEBERTA: launch_one<T, MECH_DEBERTA>(a, grid, stream); break;
    case MECH_ALIBI: launch_one<T, MECH_ALIBI>(a, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, bool fp32, hipStream_t stream) {
  return fp32 ? launch_fwd_t<float>(a, stream) : launch_fwd_t<uint16_t>(a, stream);
}

}  // namespace relpos
