"""fp64 CPU oracle for exact softmax attention with additive relative-position terms.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the bench's CPU-baseline leg do.  It
shares no code with the HIP library.

What it computes (one (batch, head) slice at a time, all in float64):

    S_ij = s * q_i . k_j + B_ij      on allowed pairs, -inf elsewhere
    P    = softmax_j(S),  O = P V,  LSE_i = ln sum_j exp(S_ij)

This is the score of "Fast and Exact Relative-Position Attention via
Structure-Aware Kernels" as restated by the zicq.com explainer, section "why
relative-position attention is hard to make fast" (score formula with the
additive B term).  The abstract (all pages) says the method is exact, so the
oracle is simply that definition written out with B materialised as an L x L
matrix.  The four mechanisms are the ones the authors list in their comment on
the Hugging Face paper page (DeBERTa, Shaw, Transformer-XL, T5); the pages do
not define them, so each B below is the plainest reading of the original
mechanism:

    T5       B_ij = beta[h, bucket(j - i)]                     (scalar bias)
    Shaw     B_ij = s * q_i . w[clamp(j - i, -k, k) + k]       (key side)
    T-XL     S_ij = s * ((q_i + u_h) . k_j + (q_i + v_h) . r_h[i - j])
    DeBERTa  S_ij = s * (q_i . k_j + q_i . Kr[c2p(i,j)] + k_j . Qr[p2c(i,j)])
             c2p(i,j) = clamp(i - j + k, 0, 2k - 1),  p2c(i,j) = clamp(j - i + k, 0, 2k - 1)
    ALiBi    B_ij = -m_h * |i - j|                             (slope per head, unscaled)

ALiBi is not one of the authors' four; the explainer names it among the models the method
suits (section on engineering trade-offs and where it applies).  Its plainest reading is the
original linear distance penalty with one slope per head, added like T5's bias; its gradient
is dm_h = -sum of dS_ij |i - j|.

Which heads share a relation table is not on the pages.  The workloads share Shaw's w and
DeBERTa's Kr, Qr across heads and give T-XL one r per head; either kind of table may instead
come with a leading head axis (one table per head) or without it (one table every head
reads).  The score of head h uses head h's table, and a shared table's gradient is the sum
over every head that reads it.

Default scale s = 1/sqrt(d), and 1/sqrt(3d) for DeBERTa.  The backward pass is
written as explicit formulas (no autograd): dV = P^T dO, dP = dO V^T,
D_i = sum_j P_ij dP_ij, dS = P * (dP - D), and every table gradient is the
scatter-sum of dS over the pairs that read that table row.  The explainer's
section on offset-based gradient sharding says many queries update the same
position parameter; here that is the plain sum over all such pairs.

Pins (tests/test_oracle_pins.py): plain attention through torch's
scaled_dot_product_attention when tables are zero, pure-Python brute force at
L <= 8, central finite differences for every gradient, bucket thresholds derived
in closed form, offset-only (Toeplitz) index maps, softmax-gradient sum
invariants, and cross-mechanism identities.
"""

from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field

import numpy as np

MECHS = ("t5", "shaw", "txl", "deberta")     # the authors' four
ALL_MECHS = MECHS + ("alibi",)


@dataclass
class Params:
    """Mechanism and mask description.

    window_left / window_right: a pair (i, j) is allowed iff
    (window_left < 0 or i - j <= window_left) and (window_right < 0 or j - i <= window_right).
    (-1, -1) is no mask, (-1, 0) is causal, (w, w) is a local window.  The pages mention
    local attention only as something offset-aware tiling must respect (zicq.com
    explainer, section "offset-aware tiling"); this rule is the plainest reading.
    """

    mech: str
    head_dim: int
    window_left: int = -1
    window_right: int = -1
    scale: float | None = None
    num_buckets: int = 32          # T5
    max_distance: int = 128        # T5
    bidirectional: bool = True     # T5
    rel_span: int = 0              # Shaw k, DeBERTa k; unused for T5 / T-XL
    extra: dict = field(default_factory=dict)

    def s(self) -> float:
        if self.scale is not None and self.scale != 0.0:
            return float(self.scale)
        if self.mech == "deberta":
            return 1.0 / math.sqrt(3.0 * self.head_dim)
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def causal(self) -> bool:
        return self.window_right == 0


# ----------------------------------------------------------------------------------
# index maps
# ----------------------------------------------------------------------------------

def t5_bucket(rel: int, num_buckets: int, max_distance: int, bidirectional: bool) -> int:
    """T5 relative-position bucket of rel = j - i (key position minus query position).

    Published T5 log-bucket map: exact buckets for small distances, then buckets whose
    width grows logarithmically up to max_distance, after which everything shares the
    last bucket.  Bidirectional maps split the buckets in two halves, the upper half for
    keys after the query.  The floor of
        max_exact + ln(n / max_exact) / ln(max_distance / max_exact) * (nb - max_exact)
    is taken in exact real arithmetic, using only integer comparisons:
        floor(x) >= t  <=>  n^E * max_exact^t >= max_distance^t * max_exact^E,
    where E = nb - max_exact.
    """
    nb = num_buckets
    ret = 0
    n = -rel                      # = i - j
    if bidirectional:
        nb //= 2
        if n < 0:
            ret += nb
        n = abs(n)
    else:
        n = max(n, 0)
    max_exact = nb // 2
    if n < max_exact:
        return ret + n
    E = nb - max_exact
    t = 0
    # largest t <= E - 1 with floor(x) >= t (the cap at nb - 1 makes larger t irrelevant)
    while t + 1 <= E - 1 and n ** E * max_exact ** (t + 1) >= max_distance ** (t + 1) * max_exact ** E:
        t += 1
    return ret + max_exact + t


def t5_bucket_by_offset(L: int, p: Params) -> np.ndarray:
    """bucket(j - i) for every offset rel = j - i in [-(L-1), L-1]; entry rel + L - 1."""
    return _t5_offset_map(L, p.num_buckets, p.max_distance, bool(p.bidirectional)).copy()


@functools.lru_cache(maxsize=16)
def _t5_offset_map(L: int, nb: int, md: int, bidir: bool) -> np.ndarray:
    return np.array([t5_bucket(rel, nb, md, bidir) for rel in range(-(L - 1), L)], dtype=np.int64)


def txl_rows(L: int, p: Params) -> int:
    """Rows of the T-XL relation table r_h.  Causal masks only ever read i - j >= 0,
    so the table holds offsets 0..L-1; otherwise offsets -(L-1)..L-1."""
    return L if p.causal else 2 * L - 1


def txl_row_of_offset(delta: np.ndarray, L: int, p: Params) -> np.ndarray:
    """Table row of offset delta = i - j for T-XL (row = delta, or delta + L - 1)."""
    return delta if p.causal else delta + (L - 1)


def allowed_mask(rows: np.ndarray, L: int, p: Params) -> np.ndarray:
    i = rows[:, None]
    j = np.arange(L)[None, :]
    ok = np.ones((len(rows), L), dtype=bool)
    if p.window_left >= 0:
        ok &= (i - j) <= p.window_left
    if p.window_right >= 0:
        ok &= (j - i) <= p.window_right
    return ok


def index_maps(rows: np.ndarray, L: int, p: Params) -> dict:
    """Per-pair table rows for query rows `rows` and all keys: int64 arrays [len(rows), L]."""
    i = rows[:, None].astype(np.int64)
    j = np.arange(L, dtype=np.int64)[None, :]
    rel = j - i                     # key minus query
    delta = i - j                   # query minus key
    if p.mech == "t5":
        table = t5_bucket_by_offset(L, p)
        return {"bucket": table[rel + (L - 1)]}
    if p.mech == "shaw":
        k = p.rel_span
        return {"row": np.clip(rel, -k, k) + k}
    if p.mech == "txl":
        return {"row": txl_row_of_offset(delta, L, p)}
    if p.mech == "deberta":
        k = p.rel_span
        return {"c2p": np.clip(delta + k, 0, 2 * k - 1), "p2c": np.clip(rel + k, 0, 2 * k - 1)}
    if p.mech == "alibi":
        return {"dist": np.abs(delta)}
    raise ValueError(p.mech)


# ----------------------------------------------------------------------------------
# scores
# ----------------------------------------------------------------------------------

def _f64(x):
    return np.asarray(x, dtype=np.float64)


# relation tables and their rank without a head axis; beta, u, v and slopes are always per head
REL_TABLE_NDIM = {"w": 2, "r": 2, "kr": 2, "qr": 2}


def has_head_axis(name: str, table) -> bool:
    """True when `table` holds one table per head (leading head axis)."""
    if name in REL_TABLE_NDIM:
        return np.ndim(table) == REL_TABLE_NDIM[name] + 1
    return True


def head_table(tables: dict, name: str, h: int) -> np.ndarray:
    """Head h's relation table (the table itself when every head shares it)."""
    t = _f64(tables[name])
    return t[h] if has_head_axis(name, t) else t


def bias_rows(p: Params, q: np.ndarray, k: np.ndarray, tables: dict, h: int,
              rows: np.ndarray) -> np.ndarray:
    """Materialised additive term B[rows, :] for one (batch, head): q, k are [L, d]."""
    L = k.shape[0]
    s = p.s()
    idx = index_maps(rows, L, p)
    if p.mech == "t5":
        beta = _f64(tables["beta"])[h]
        return beta[idx["bucket"]]
    if p.mech == "shaw":
        w = head_table(tables, "w", h)
        G = q[rows] @ w.T                                   # [rows, 2k+1]: q_i . w_c
        return s * np.take_along_axis(G, idx["row"], axis=1)
    if p.mech == "txl":
        r = head_table(tables, "r", h)
        v = _f64(tables["v"])[h]
        u = _f64(tables["u"])[h]
        G = (q[rows] + v) @ r.T                             # [rows, Nrel]: (q_i + v) . r_c
        pos = s * np.take_along_axis(G, np.clip(idx["row"], 0, r.shape[0] - 1), axis=1)
        pos = np.where((idx["row"] >= 0) & (idx["row"] < r.shape[0]), pos, 0.0)
        content_u = s * (k @ u)[None, :]                    # s * u . k_j
        return pos + content_u
    if p.mech == "deberta":
        kr = head_table(tables, "kr", h)
        qr = head_table(tables, "qr", h)
        G1 = q[rows] @ kr.T                                 # [rows, 2k]: q_i . Kr_c
        G2 = k @ qr.T                                       # [L, 2k]:    k_j . Qr_c
        c2p = np.take_along_axis(G1, idx["c2p"], axis=1)
        p2c = G2[np.arange(L)[None, :], idx["p2c"]]
        return s * (c2p + p2c)
    if p.mech == "alibi":
        m = float(_f64(tables["slopes"])[h])
        return -m * idx["dist"].astype(np.float64)
    raise ValueError(p.mech)


def scores_rows(p: Params, q: np.ndarray, k: np.ndarray, tables: dict, h: int,
                rows: np.ndarray) -> np.ndarray:
    """S[rows, :] for one (batch, head), -inf on disallowed pairs."""
    L = k.shape[0]
    S = p.s() * (q[rows] @ k.T) + bias_rows(p, q, k, tables, h, rows)
    S = np.where(allowed_mask(rows, L, p), S, -np.inf)
    return S


def _softmax_rows(S: np.ndarray):
    m = np.max(S, axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    e = np.exp(S - m)
    l = np.sum(e, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(empty, 0.0, e / np.where(l == 0, 1.0, l))
        lse = np.where(empty[:, 0], -np.inf, m[:, 0] + np.log(np.where(l[:, 0] == 0, 1.0, l[:, 0])))
    return P, lse


# ----------------------------------------------------------------------------------
# forward / backward
# ----------------------------------------------------------------------------------

def forward_rows(p: Params, q, k, v, tables: dict, b: int, h: int, rows=None):
    """O[rows] and LSE[rows] of one (batch, head).  q, k, v: [B, H, L, d]."""
    L = q.shape[2]
    if rows is None:
        rows = np.arange(L)
    rows = np.asarray(rows, dtype=np.int64)
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    S = scores_rows(p, qh, kh, tables, h, rows)
    P, lse = _softmax_rows(S)
    return P @ vh, lse


def forward(p: Params, q, k, v, tables: dict):
    """O [B, H, L, d] and LSE [B, H, L] in float64."""
    B, H, L, d = q.shape
    O = np.zeros((B, H, L, d))
    LSE = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = forward_rows(p, q, k, v, tables, b, h)
    return O, LSE


def table_shapes(p: Params, H: int, L: int, d: int) -> dict:
    if p.mech == "t5":
        return {"beta": (H, p.num_buckets)}
    if p.mech == "shaw":
        return {"w": (2 * p.rel_span + 1, d)}
    if p.mech == "txl":
        return {"r": (H, txl_rows(L, p), d), "u": (H, d), "v": (H, d)}
    if p.mech == "deberta":
        return {"kr": (2 * p.rel_span, d), "qr": (2 * p.rel_span, d)}
    if p.mech == "alibi":
        return {"slopes": (H,)}
    raise ValueError(p.mech)


def _pair_scatter(dS: np.ndarray, idx: np.ndarray, ntab: int, by_key: bool = False) -> np.ndarray:
    """N[a, c] = sum over pairs with table row idx == c of dS, grouped by query a = i
    (or by key a = j when by_key).  This is the plain per-row scatter-sum."""
    L_i, L_j = dS.shape
    if by_key:
        a = np.broadcast_to(np.arange(L_j)[None, :], dS.shape)
        n_a = L_j
    else:
        a = np.broadcast_to(np.arange(L_i)[:, None], dS.shape)
        n_a = L_i
    valid = (idx >= 0) & (idx < ntab)
    flat = (a * ntab + np.where(valid, idx, 0)).ravel()
    w = np.where(valid, dS, 0.0).ravel()
    return np.bincount(flat, weights=w, minlength=n_a * ntab).reshape(n_a, ntab)


def backward_head(p: Params, q, k, v, tables: dict, dO, b: int, h: int):
    """Gradients for one (batch, head): dq, dk, dv [L, d] and this slice's table grads."""
    L = q.shape[2]
    s = p.s()
    rows = np.arange(L)
    qh, kh, vh, doh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(dO[b, h])
    S = scores_rows(p, qh, kh, tables, h, rows)
    P, _ = _softmax_rows(S)
    dV = P.T @ doh
    dP = doh @ vh.T
    D = np.sum(P * dP, axis=1)
    dS = P * (dP - D[:, None])
    idx = index_maps(rows, L, p)
    g = {}
    if p.mech == "t5":
        dq = s * (dS @ kh)
        dk = s * (dS.T @ qh)
        nb = p.num_buckets
        g["beta"] = np.bincount(idx["bucket"].ravel(), weights=dS.ravel(), minlength=nb)
    elif p.mech == "shaw":
        w = head_table(tables, "w", h)
        N = _pair_scatter(dS, idx["row"], w.shape[0])
        dq = s * (dS @ kh) + s * (N @ w)
        dk = s * (dS.T @ qh)
        g["w"] = s * (N.T @ qh)
    elif p.mech == "txl":
        r = head_table(tables, "r", h)
        u = _f64(tables["u"])[h]
        vv = _f64(tables["v"])[h]
        N = _pair_scatter(dS, idx["row"], r.shape[0])
        dq = s * (dS @ kh) + s * (N @ r)
        dk = s * (dS.T @ (qh + u))
        g["r"] = s * (N.T @ (qh + vv))
        g["u"] = s * np.sum(dS @ kh, axis=0)
        g["v"] = s * np.sum(N @ r, axis=0)
    elif p.mech == "deberta":
        kr = head_table(tables, "kr", h)
        qr = head_table(tables, "qr", h)
        N1 = _pair_scatter(dS, idx["c2p"], kr.shape[0])
        N2 = _pair_scatter(dS, idx["p2c"], qr.shape[0], by_key=True)
        dq = s * (dS @ kh) + s * (N1 @ kr)
        dk = s * (dS.T @ qh) + s * (N2 @ qr)
        g["kr"] = s * (N1.T @ qh)
        g["qr"] = s * (N2.T @ kh)
    elif p.mech == "alibi":
        dq = s * (dS @ kh)
        dk = s * (dS.T @ qh)
        g["slopes"] = -np.sum(dS * idx["dist"])
    else:
        raise ValueError(p.mech)
    return dq, dk, dV, g


def dq_rows(p: Params, q, k, v, tables: dict, dO, b: int, h: int, rows):
    """dQ at the given query rows of one (batch, head): the query-side gradient restricted
    to those rows (same formulas as backward_head, whose row i depends only on row i of S,
    P and dP).  Cheap at any length: O(len(rows) * L * d)."""
    L = q.shape[2]
    s = p.s()
    rows = np.asarray(rows, dtype=np.int64)
    qh, kh, vh, doh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(dO[b, h])
    S = scores_rows(p, qh, kh, tables, h, rows)
    P, _ = _softmax_rows(S)
    dP = doh[rows] @ vh.T
    D = np.sum(P * dP, axis=1)
    dS = P * (dP - D[:, None])
    idx = index_maps(rows, L, p)
    dq = s * (dS @ kh)
    if p.mech == "shaw":
        w = head_table(tables, "w", h)
        dq += s * (_pair_scatter(dS, idx["row"], w.shape[0]) @ w)
    elif p.mech == "txl":
        r = head_table(tables, "r", h)
        dq += s * (_pair_scatter(dS, idx["row"], r.shape[0]) @ r)
    elif p.mech == "deberta":
        kr = head_table(tables, "kr", h)
        dq += s * (_pair_scatter(dS, idx["c2p"], kr.shape[0]) @ kr)
    elif p.mech not in ("t5", "alibi"):
        raise ValueError(p.mech)
    return dq


def add_table_grads(grads: dict, g: dict, tables: dict, h: int) -> None:
    """Add one (batch, head) slice's table gradients g into grads: per-head tables at their
    head, shared tables summed over heads."""
    for name, val in g.items():
        if has_head_axis(name, tables[name]):
            grads[name][h] += val
        else:
            grads[name] += val


def backward_chunk(p: Params, q, k, v, tables: dict, dO, b: int, h: int, rows) -> dict:
    """The part of one (batch, head)'s backward that comes from the query rows `rows`: the same
    formulas as backward_head on those rows of S, P, dP and dS.  Each row's softmax, dP and D
    depend on that row only, so they are whole; returns dq at those rows and the rows'
    contributions to every sum over query rows (dK, dV, table gradients, and DeBERTa's p2c
    scatter grouped by key, which finish_chunks turns into dK and dQr)."""
    L = q.shape[2]
    s = p.s()
    rows = np.asarray(rows, dtype=np.int64)
    qh, kh, vh, doh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(dO[b, h])
    qc, doc = qh[rows], doh[rows]
    S = scores_rows(p, qh, kh, tables, h, rows)
    P, lse = _softmax_rows(S)
    dP = doc @ vh.T
    D = np.sum(P * dP, axis=1)
    dS = P * (dP - D[:, None])
    idx = index_maps(rows, L, p)
    # the forward outputs of these rows come with them (as forward_rows forms them)
    out = {"rows": rows, "o": P @ vh, "lse": lse, "dv": P.T @ doc}
    dqc = s * (dS @ kh)
    g = {}
    if p.mech == "t5":
        out["dk"] = s * (dS.T @ qc)
        g["beta"] = np.bincount(idx["bucket"].ravel(), weights=dS.ravel(), minlength=p.num_buckets)
    elif p.mech == "shaw":
        w = head_table(tables, "w", h)
        N = _pair_scatter(dS, idx["row"], w.shape[0])
        dqc += s * (N @ w)
        out["dk"] = s * (dS.T @ qc)
        g["w"] = s * (N.T @ qc)
    elif p.mech == "txl":
        r = head_table(tables, "r", h)
        u = _f64(tables["u"])[h]
        vv = _f64(tables["v"])[h]
        N = _pair_scatter(dS, idx["row"], r.shape[0])
        dqc += s * (N @ r)
        out["dk"] = s * (dS.T @ (qc + u))
        g["r"] = s * (N.T @ (qc + vv))
        g["u"] = s * np.sum(dS @ kh, axis=0)
        g["v"] = s * np.sum(N @ r, axis=0)
    elif p.mech == "deberta":
        kr = head_table(tables, "kr", h)
        qr = head_table(tables, "qr", h)
        N1 = _pair_scatter(dS, idx["c2p"], kr.shape[0])
        dqc += s * (N1 @ kr)
        out["dk"] = s * (dS.T @ qc)
        g["kr"] = s * (N1.T @ qc)
        out["n2"] = _pair_scatter(dS, idx["p2c"], qr.shape[0], by_key=True)
    elif p.mech == "alibi":
        out["dk"] = s * (dS.T @ qc)
        g["slopes"] = -np.sum(dS * idx["dist"])
    else:
        raise ValueError(p.mech)
    out["dq"] = dqc
    out["g"] = g
    return out


def sum_chunks(parts) -> dict:
    """Merge backward_chunk parts (disjoint row sets) into one part, summing in the order given."""
    out = None
    for part in parts:
        if out is None:
            out = {"rows": part["rows"], "dq": part["dq"], "o": part["o"], "lse": part["lse"],
                   "dk": part["dk"].copy(), "dv": part["dv"].copy(),
                   "g": {n: np.copy(v) for n, v in part["g"].items()}}
            if "n2" in part:
                out["n2"] = part["n2"].copy()
            continue
        for n in ("rows", "dq", "o", "lse"):
            out[n] = np.concatenate([out[n], part[n]])
        out["dk"] += part["dk"]
        out["dv"] += part["dv"]
        for n, v in part["g"].items():
            out["g"][n] = out["g"][n] + v
        if "n2" in part:
            out["n2"] += part["n2"]
    return out


def finish_chunks(p: Params, k, tables: dict, b: int, h: int, part: dict) -> tuple:
    """dq, dk, dv [L, d] and the slice's table gradients, as backward_head returns them, from the
    merged part of every query row (DeBERTa's p2c terms need the scatter of all rows)."""
    L, d = k.shape[2], k.shape[3]
    s = p.s()
    dq = np.zeros((L, d))
    dq[part["rows"]] = part["dq"]
    dk = part["dk"].copy()
    g = dict(part["g"])
    if p.mech == "deberta":
        qr = head_table(tables, "qr", h)
        dk += s * (part["n2"] @ qr)
        g["qr"] = s * (part["n2"].T @ _f64(k[b, h]))
    return dq, dk, part["dv"], g


def row_chunks(L: int, chunk: int):
    """Consecutive query-row ranges of at most `chunk` rows covering 0 .. L - 1."""
    return [np.arange(r0, min(L, r0 + chunk)) for r0 in range(0, L, chunk)]


def backward_head_chunked(p: Params, q, k, v, tables: dict, dO, b: int, h: int,
                          chunk: int = 512):
    """backward_head for long sequences: the query rows `chunk` at a time (backward_chunk), so
    that no L x L matrix is held, summed in ascending row order (sum_chunks, finish_chunks)."""
    parts = [backward_chunk(p, q, k, v, tables, dO, b, h, rows)
             for rows in row_chunks(q.shape[2], chunk)]
    return finish_chunks(p, k, tables, b, h, sum_chunks(parts))


def backward(p: Params, q, k, v, tables: dict, dO):
    """Full backward: dq, dk, dv [B, H, L, d] and table gradients (summed over every
    (batch, head) that reads the table; per-head tables keep their head axis)."""
    B, H, L, d = q.shape
    dq = np.zeros((B, H, L, d))
    dk = np.zeros((B, H, L, d))
    dv = np.zeros((B, H, L, d))
    grads = {name: np.zeros(np.shape(t)) for name, t in tables.items()}
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], g = backward_head(p, q, k, v, tables, dO, b, h)
            add_table_grads(grads, g, tables, h)
    return dq, dk, dv, grads
