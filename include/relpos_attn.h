/*
 * relpos_attn.h -- C ABI of the MI355X (gfx950) exact relative-position attention library.
 *
 * Operation.  For every batch b and head h, with query i and key j (0 <= i, j < L),
 *
 *     S_ij = s * q_i . k_j + B_ij          (pairs outside the mask are -inf)
 *     O    = softmax_j(S) V,   LSE_i = ln sum_j exp(S_ij)
 *
 * the score of "Fast and Exact Relative-Position Attention via Structure-Aware Kernels"
 * (zicq.com explainer, section on why relative-position attention is hard to make fast),
 * computed exactly and without ever forming the L x L term B (abstract: exact attention with
 * additive relative-position terms folded into FlashAttention-style tiling).  The four B terms
 * are the mechanisms the authors list in their comment on the Hugging Face paper page:
 *
 *   RELPOS_T5       B_ij = beta[h][bucket(j - i)]                        (bias_a = beta)
 *   RELPOS_SHAW     B_ij = s q_i . w[clamp(j - i, -k, k) + k]           (rel_a = w)
 *   RELPOS_TXL      S_ij = s ((q_i + u_h) . k_j + (q_i + v_h) . r_h[row(i - j)])
 *                   (rel_a = r, bias_a = u, bias_b = v)
 *   RELPOS_DEBERTA  S_ij = s (q_i . k_j + q_i . Kr[clamp(i - j + k, 0, 2k - 1)]
 *                                       + k_j . Qr[clamp(j - i + k, 0, 2k - 1)])
 *                   (rel_a = Kr, rel_b = Qr)
 *   RELPOS_ALIBI    B_ij = -m_h |i - j|                                  (bias_a = m)
 *
 * ALiBi is a fifth, scalar-offset mechanism: the zicq.com explainer names it among the models
 * the method suits (section on engineering trade-offs and where it applies); the authors do
 * not list it.  Its term is the linear distance penalty with one slope per head, added
 * unscaled like T5's bias.
 * T5 buckets follow the published T5 log-bucket map with an exact floor (bidirectional maps put
 * keys after the query in the upper half).  T-XL tables hold offsets 0..L-1 (row = i - j) when
 * the mask is causal (window_right == 0) and -(L-1)..L-1 (row = i - j + L - 1) otherwise.
 * Default scale s: 1/sqrt(d), and 1/sqrt(3d) for DeBERTa.
 *
 * Mask: pair (i, j) is allowed iff (window_left < 0 || i - j <= window_left) and
 * (window_right < 0 || j - i <= window_right).  (-1,-1) none, (-1,0) causal, (w,w) local.
 *
 * Layouts (row-major, last index fastest, no padding):
 *   q, k, v, o, dout, dq, dk, dv : [batch, heads, seqlen, head_dim], element type `dtype`
 *   lse                          : [batch, heads, seqlen] float (natural log)
 *   T5 beta  [heads, num_buckets] float        T-XL u, v  [heads, head_dim] float
 *   ALiBi m  [heads] float
 *   relation tables (dtype), one per head or one shared by every head (rel_head_stride):
 *     Shaw w [2k+1, head_dim]    T-XL r [Nrel, head_dim]    DeBERTa Kr, Qr [2k, head_dim]
 * Every table gradient is float and is OVERWRITTEN (not accumulated): beta, u, v and m have
 * their table's shape; a relation table's gradient is [heads, rows, head_dim] (dense) when the
 * tables are per head and [rows, head_dim] when one table is shared, the sum over every
 * (batch, head) that reads it.  Unused table / gradient slots must be NULL.
 *
 * Ownership: the caller owns every buffer, including the workspace (size it with
 * relpos_attn_workspace_size).  The library never allocates device memory.  All device
 * pointers must be 16-byte aligned, the workspace 256-byte aligned.  Work is enqueued on
 * `stream` (NULL = the default stream) and the call returns without
 * synchronising.  Results are bitwise deterministic: every sum is taken in a fixed order (the
 * few atomic adds, see relpos_attn_bwd, reach each address once per launch, launches in stream
 * order).
 *
 * Errors: every entry point returns RELPOS_OK (0) or a negative status; on error nothing has
 * been launched.  RELPOS_E_LAUNCH reports a failed kernel launch (work already enqueued by the
 * same call may have run).  relpos_status_string() names a status.
 */
#ifndef RELPOS_ATTN_H
#define RELPOS_ATTN_H

#include <stddef.h>
#include <stdint.h>

/* HIP's stream and event handles, declared as HIP's runtime header declares them (opaque
 * pointers), so that this header also compiles without the HIP headers; a repeated identical
 * typedef is valid C11 and C++. */
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RELPOS_T5 = 0, RELPOS_SHAW = 1, RELPOS_TXL = 2, RELPOS_DEBERTA = 3,
  RELPOS_ALIBI = 4  /* B_ij = -m_h |i - j| with per-head slopes m (bias_a, fp32 [H]), unscaled */
} relpos_mech;
typedef enum { RELPOS_BF16 = 0, RELPOS_FP32 = 1 } relpos_dtype;

enum {
  RELPOS_OK = 0,
  RELPOS_E_INVALID = -1,     /* bad enum, shape, NULL / misaligned pointer, span inconsistent */
  RELPOS_E_UNSUPPORTED = -2, /* valid request outside what the kernels implement: head_dim != 64,
                                 or a sequence or table too long for the kernels' 32-bit
                                 in-slice offsets: max(seqlen, table rows) * 64 * element size
                                 must stay below 2^32 bytes */
  RELPOS_E_WORKSPACE = -3,   /* workspace NULL or smaller than relpos_attn_workspace_size() */
  RELPOS_E_LAUNCH = -4       /* a kernel launch failed */
};

typedef struct relpos_desc {
  int32_t mech;           /* relpos_mech */
  int32_t dtype;          /* relpos_dtype of q, k, v, o, dout, dq, dk, dv and rel_a / rel_b */
  int64_t batch;          /* >= 0 (0 = nothing to do) */
  int64_t heads;          /* >= 1 */
  int64_t seqlen;         /* L >= 0, queries and keys alike */
  int64_t head_dim;       /* d; the kernels implement d = 64 */
  int32_t window_left;    /* -1 = unbounded */
  int32_t window_right;   /* -1 = unbounded; 0 = causal */
  int32_t rel_span;       /* Shaw / DeBERTa k >= 1; ignored for T5 and T-XL */
  int32_t num_buckets;    /* T5: even when bidirectional, >= 2 per direction */
  int32_t max_distance;   /* T5: > num_buckets / 4 (bidirectional) or num_buckets / 2 */
  int32_t bidirectional;  /* T5: 1 = separate buckets for keys after the query */
  float scale;            /* 0 = default */
  int64_t max_partial_bytes; /* T-XL backward: the key-side r partials take L^2 / 2 bytes per
                                (batch, head) slice, so the key-side pass runs over fixed groups
                                of slices, each group's partials summed into dr before the next
                                reuses them.  0 = groups of as many slices as give 512 workgroups
                                (one full wave on an MI355X; L = 8192: 8 slices, 1.1 GB);
                                > 0 = as many slices as fit in this many bytes.  At least one
                                slice per group.  Results depend on the group size only through
                                the (fixed) order of the fp32 sums. */
  int64_t rel_head_stride;   /* elements between the relation tables (rel_a, rel_b) of
                                consecutive heads: 0 = one table shared by every head; otherwise
                                head h reads rel_a + h * rel_head_stride (and rel_b likewise),
                                with rel_head_stride >= rows * head_dim and a multiple of 8.  The
                                workloads of the pages share Shaw's w and DeBERTa's Kr / Qr
                                (stride 0) and give T-XL one r per head (stride Nrel * 64).
                                Ignored for T5 and ALiBi, whose tables are per head. */
} relpos_desc;

/* Bytes of workspace the forward (pass 0) or backward (pass 1) call needs. */
int relpos_attn_workspace_size(const relpos_desc* desc, int pass, size_t* bytes);

/* Forward: writes O and LSE. */
int relpos_attn_fwd(const relpos_desc* desc, const void* q, const void* k, const void* v,
                    const void* rel_a, const void* rel_b, const float* bias_a,
                    const float* bias_b, void* o, float* lse, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* Backward from (q, k, v, o, lse, dout): writes dq, dk, dv and the table gradients
 * (T5: dbias_a = dbeta; Shaw: drel_a = dw; T-XL: drel_a = dr, dbias_a = du, dbias_b = dv;
 * DeBERTa: drel_a = dKr, drel_b = dQr; ALiBi: dbias_a = dm, the slopes' gradient), with
 * dS = P (dP - D), D_i = dO_i . O_i, and every table gradient the sum of dS-weighted operands
 * over the pairs that read each table row.  Offset-based gradient sharding (abstract of "Fast and
 * Exact Relative-Position Attention via Structure-Aware Kernels", item 3; zicq.com explainer,
 * section on how structure-aware tiling stays exact, part 3, offset-based gradient sharding):
 * each workgroup reduces dS along the diagonals of its own tiles into an offset-indexed partial
 * of its own, and a second pass sums the partials of every (batch, head) that reads a table row
 * in a fixed order, so the result is bitwise reproducible.  (Shaw and DeBERTa at large B H L:
 * the batch entries of a head run in turn, one launch each, into one partial; the first launch
 * stores it and each later one adds to it with one atomic add per element, so every element's
 * sum still has one fixed order.)  T5 sums dS per bucket inside the workgroup.  bf16, or
 * fp32 (every matrix-core operand split into two bf16 parts, hi and lo, with the products
 * hi.hi + hi.lo + lo.hi accumulated in fp32).  The workspace (relpos_attn_workspace_size,
 * pass 1) holds the partials; its size grows with B H L (T-XL: L^2 / 2 bytes for each
 * (batch, head) slice of one group, see max_partial_bytes). */
int relpos_attn_bwd(const relpos_desc* desc, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dout, const void* rel_a,
                    const void* rel_b, const float* bias_a, const float* bias_b, void* dq,
                    void* dk, void* dv, float* drel_a, float* drel_b, float* dbias_a,
                    float* dbias_b, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The forward for callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation): the same kernels and results as
 * relpos_attn_fwd, with the workspace in a device array of RELPOS_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  The call allocates nothing; the
 * caller passes inputs and outputs as for relpos_attn_fwd.  A problem whose forward workspace
 * (relpos_attn_workspace_size, pass 0) exceeds RELPOS_NOALLOC_SCRATCH_BYTES is refused with
 * RELPOS_E_WORKSPACE before any launch.  Every call on one GPU shares that GPU's array and
 * leaves its contents behind (nothing in it needs to start at zero: each call rewrites what it
 * reads), so calls that overlap on one GPU (several streams or threads at once) race: serialise
 * them.  The first call on each device looks up the array's device address (hipGetSymbolAddress)
 * with that device current; RELPOS_E_LAUNCH if that fails. */
#define RELPOS_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int relpos_attn_fwd_noalloc(const relpos_desc* desc, const void* q, const void* k, const void* v,
                            const void* rel_a, const void* rel_b, const float* bias_a,
                            const float* bias_b, void* o, float* lse, hipStream_t stream);

/* Index maps the kernels use, computed on the device: for every offset delta = i - j in
 * [-(L-1), L-1], out_a[delta + L - 1] is the table row of that offset (T5 bucket, Shaw row,
 * T-XL row or -1 when the table has no such row, DeBERTa c2p row, ALiBi distance |delta|)
 * and, for DeBERTa only,
 * out_b[delta + L - 1] is the p2c row (out_b must be NULL otherwise).  Both int32 device
 * buffers of 2L - 1 entries. */
int relpos_index_map(const relpos_desc* desc, int32_t* out_a, int32_t* out_b,
                     hipStream_t stream);

/* Relation-table projections.  The T-XL table r and the DeBERTa tables Kr, Qr are projections
 * of a position basis in the original mechanisms (T-XL: r = R W_r, R the sinusoid features of
 * every offset; DeBERTa: Kr = P W_r^k and Qr = P W_r^q); the zicq.com explainer's section on
 * reusing query-key relation products covers these "basis times weight" terms.  With X the basis
 * [N, F] and W [F, H d] (head h owns columns h d .. h d + d - 1):
 *
 *   relpos_project_fwd   rel[h][n][c] = sum_f X[n][f] W[f][h d + c]        -> [H, N, d], dtype
 *   relpos_project_bwd   dX[n][f]     = sum_{h,c} drel[h][n][c] W[f][h d + c]   [N, F] float
 *                        dW[f][h d+c] = sum_n X[n][f] drel[h][n][c]             [F, H d] float
 *
 * rel has exactly the layout relpos_attn_fwd reads for rel_a / rel_b (T-XL: H heads, N = Nrel;
 * DeBERTa: H = 1, N = 2k), and drel the layout relpos_attn_bwd writes for drel_a / drel_b, so the
 * projection chains with the attention calls without copies.  DeBERTa's two tables come from one
 * call with W = [W_r^k | W_r^q] as two heads (Kr = rel[0], Qr = rel[1]); when relpos_attn_bwd
 * writes drel_a and drel_b into the two halves of one [2, 2k, d] buffer, one backward call
 * gives dP summed over both projections and [dW_r^k | dW_r^q].  Products run on the matrix cores
 * with fp32 accumulation; fp32 operands are split into two bf16 parts (three products), giving
 * close to fp32 accuracy.  dW is reduced over n in fixed slices, in a fixed order (deterministic);
 * the slices' partial sums live in the workspace (relpos_project_workspace_size; may be 0).
 * Either of dX / dW may be NULL (not computed; T-XL's R is fixed, so dX is usually not needed).
 * Outputs are OVERWRITTEN.  Requirements: 0 <= N <= 2^24, 8 <= F <= 65536 and 8 <= d with F, d
 * multiples of 8, H d <= 65536; every pointer 16-byte aligned, the workspace 256-byte aligned.
 * Ownership, streams and errors as for the attention calls. */
typedef struct relpos_proj_desc {
  int32_t dtype;        /* relpos_dtype of X, W and rel */
  int64_t rows;         /* N: basis rows */
  int64_t in_features;  /* F */
  int64_t heads;        /* H */
  int64_t head_dim;     /* d */
} relpos_proj_desc;

int relpos_project_fwd(const relpos_proj_desc* desc, const void* X, const void* W, void* rel,
                       hipStream_t stream);
int relpos_project_workspace_size(const relpos_proj_desc* desc, size_t* bytes);
int relpos_project_bwd(const relpos_proj_desc* desc, const void* X, const void* W,
                       const float* drel, float* dX, float* dW, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Profiling hook for benchmarks.  When `kernel` is RELPOS_PROF_FWD, RELPOS_PROF_BWD_DQ or
 * RELPOS_PROF_BWD_DKDV, later calls made BY THE SAME HOST THREAD record `start_event` on their
 * stream just before enqueueing that pass and `stop_event` just after its last launch (both
 * created by the caller).  A pass may be several launches (the light and general
 * parts of Shaw and DeBERTa, folded batch entries); the T-XL key-side pass under
 * max_partial_bytes also spans the aggregations between its slice groups.  RELPOS_PROF_OFF (0) clears the hook.  The setting is thread-local:
 * calls from other threads never see it, so the library stays safe to call from several
 * threads on their own streams.  Returns RELPOS_E_INVALID for an unknown kernel id or NULL
 * events. */
enum { RELPOS_PROF_OFF = 0, RELPOS_PROF_FWD = 1, RELPOS_PROF_BWD_DQ = 2, RELPOS_PROF_BWD_DKDV = 3 };
int relpos_profile_events(hipEvent_t start_event, hipEvent_t stop_event, int kernel);

/* Static string naming a status code. */
const char* relpos_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int relpos_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RELPOS_ATTN_H */
