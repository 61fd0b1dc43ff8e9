"""Scalar-loop brute force of the same attention, for tiny inputs (L <= 8).

TEST INFRASTRUCTURE ONLY (see relpos_oracle).  It re-derives every score term pair
by pair with plain Python floats and math.log / math.exp, so that a vectorisation
or indexing slip in relpos_oracle (a transposed gather, a wrong table row, a sign
error in an offset) shows up as a disagreement.  The T5 bucket here uses the
floating-point logarithm of the published T5 map (truncated toward zero) rather
than the integer comparison used by relpos_oracle; both must agree on every
offset the tests use.
"""

from __future__ import annotations

import math


def _bucket_float(rel, nb, md, bidir):
    n = -rel
    ret = 0
    if bidir:
        nb //= 2
        if n < 0:
            ret += nb
        n = abs(n)
    else:
        n = max(n, 0)
    me = nb // 2
    if n < me:
        return ret + n
    large = me + int(math.log(n / me) / math.log(md / me) * (nb - me))
    return ret + min(large, nb - 1)


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def _clamp(x, lo, hi):
    return lo if x < lo else hi if x > hi else x


def _head_rows(tab, h):
    """Head h's table: tab is a list of rows, or a list of per-head lists of rows."""
    return tab[h] if isinstance(tab[0][0], list) else tab


def score(p, q, k, tables, h, i, j):
    """S_ij for one (batch, head); q, k are lists of rows (lists of floats)."""
    L = len(k)
    if p.window_left >= 0 and i - j > p.window_left:
        return -math.inf
    if p.window_right >= 0 and j - i > p.window_right:
        return -math.inf
    s = p.s()
    qi, kj = q[i], k[j]
    if p.mech == "t5":
        beta = tables["beta"][h]
        return s * _dot(qi, kj) + float(beta[_bucket_float(j - i, p.num_buckets, p.max_distance,
                                                             p.bidirectional)])
    if p.mech == "shaw":
        kk = p.rel_span
        w = _head_rows(tables["w"], h)[_clamp(j - i, -kk, kk) + kk]
        return s * _dot(qi, kj) + s * _dot(qi, w)
    if p.mech == "txl":
        u = tables["u"][h]
        v = tables["v"][h]
        row = (i - j) if p.window_right == 0 else (i - j) + (L - 1)
        r = _head_rows(tables["r"], h)[row]
        qu = [a + c for a, c in zip(qi, u)]
        qv = [a + c for a, c in zip(qi, v)]
        return s * _dot(qu, kj) + s * _dot(qv, r)
    if p.mech == "deberta":
        kk = p.rel_span
        kr = _head_rows(tables["kr"], h)[_clamp(i - j + kk, 0, 2 * kk - 1)]
        qr = _head_rows(tables["qr"], h)[_clamp(j - i + kk, 0, 2 * kk - 1)]
        return s * (_dot(qi, kj) + _dot(qi, kr) + _dot(kj, qr))
    if p.mech == "alibi":
        return s * _dot(qi, kj) - float(tables["slopes"][h]) * abs(i - j)
    raise ValueError(p.mech)


def forward_head(p, q, k, v, tables, h):
    """O (list of rows) and LSE (list) for one (batch, head), by scalar loops."""
    L = len(q)
    d = len(v[0])
    O, LSE = [], []
    for i in range(L):
        row = [score(p, q, k, tables, h, i, j) for j in range(L)]
        m = max(row)
        if m == -math.inf:
            O.append([0.0] * d)
            LSE.append(-math.inf)
            continue
        e = [math.exp(x - m) for x in row]
        tot = sum(e)
        O.append([sum(e[j] * v[j][c] for j in range(L)) / tot for c in range(d)])
        LSE.append(m + math.log(tot))
    return O, LSE
