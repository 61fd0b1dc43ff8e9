"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what it pins.  None of them calls the HIP library.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import projection as prj
from oracle import relpos_oracle as orc
from exact_attention_relative_amd.inputs import make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MASKS = {"none": (-1, -1), "causal": (-1, 0), "local": (2, 1)}


def _case(mech, L=7, d=4, B=1, H=2, window=(-1, -1), seed=11, span=3, nb=8, md=12,
          bidir=None, table_std=0.7, dtype="fp32"):
    c = make_case(mech, B, H, L, d, dtype=dtype, window=window, seed=seed, rel_span=span,
                  num_buckets=nb, max_distance=md, bidirectional=bidir, table_std=table_std)
    p = orc.Params(**c["params"])
    return c, p


def _f64(c):
    return (c["q"].astype(np.float64), c["k"].astype(np.float64), c["v"].astype(np.float64),
            {n: t.astype(np.float64) for n, t in c["tables"].items()}, c["dout"].astype(np.float64))


# ------------------------------------------------------------------------ T5 buckets

def _golden_buckets():
    rows = []
    with open(os.path.join(GOLDEN, "t5_buckets.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            nb, md, bd, rel, exp = (int(x) for x in line.split())
            rows.append((nb, md, bool(bd), rel, exp))
    return rows


@pytest.mark.parametrize("nb,md,bidir,rel,expected", _golden_buckets())
def test_t5_bucket_closed_form(nb, md, bidir, rel, expected):
    """Pin: hand-derived bucket thresholds, including exact power-of-two boundaries."""
    assert orc.t5_bucket(rel, nb, md, bidir) == expected


@pytest.mark.parametrize("nb,md,bidir", [(32, 128, True), (32, 1024, True), (32, 128, False),
                                         (16, 64, True), (64, 512, False)])
def test_t5_bucket_matches_float_log_form(nb, md, bidir):
    """Pin: the integer-comparison floor equals the floating-point log form of the published
    map on every offset |rel| < 8192 used by the workloads."""
    for rel in range(-8191, 8192):
        assert orc.t5_bucket(rel, nb, md, bidir) == brute._bucket_float(rel, nb, md, bidir), rel


def test_t5_bucket_monotone_and_range():
    """Pin: magnitude buckets never decrease with distance and stay inside the table."""
    for bidir in (True, False):
        prev = -1
        for n in range(0, 9000):
            b = orc.t5_bucket(-n, 32, 1024, bidir)
            assert 0 <= b < 32
            assert b >= prev
            prev = b


# ------------------------------------------------------------------------ index maps

@pytest.mark.parametrize("mech", orc.ALL_MECHS)
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_index_maps_depend_only_on_offset(mech, mask):
    """Pin: every table index is a function of i - j alone (idx[i][j] == idx[i+1][j+1])."""
    L = 40
    p = orc.Params(mech=mech, head_dim=8, window_left=MASKS[mask][0], window_right=MASKS[mask][1],
                   num_buckets=16, max_distance=20, bidirectional=(mask == "none"), rel_span=5)
    maps = orc.index_maps(np.arange(L), L, p)
    for name, m in maps.items():
        assert np.array_equal(m[1:, 1:], m[:-1, :-1]), name


def test_index_map_clamps_closed_form():
    """Pin: clamp rows written out at the ends of the span."""
    L, k = 20, 4
    p = orc.Params(mech="shaw", head_dim=8, rel_span=k)
    row = orc.index_maps(np.arange(L), L, p)["row"]
    assert row[10, 10] == k and row[10, 11] == k + 1 and row[10, 9] == k - 1
    assert row[10, 14] == 2 * k and row[10, 19] == 2 * k and row[10, 6] == 0 and row[10, 0] == 0
    p = orc.Params(mech="deberta", head_dim=8, rel_span=k)
    m = orc.index_maps(np.arange(L), L, p)
    # c2p row = clamp(i - j + k, 0, 2k-1); p2c row = clamp(j - i + k, 0, 2k-1)
    assert m["c2p"][10, 10] == k and m["c2p"][10, 9] == k + 1 and m["c2p"][10, 11] == k - 1
    assert m["c2p"][10, 0] == 2 * k - 1 and m["c2p"][10, 14] == 0
    assert m["p2c"][10, 10] == k and m["p2c"][10, 11] == k + 1 and m["p2c"][10, 19] == 2 * k - 1
    p = orc.Params(mech="txl", head_dim=8, window_right=0)
    row = orc.index_maps(np.arange(L), L, p)["row"]
    assert row[10, 3] == 7 and row[10, 10] == 0
    p = orc.Params(mech="txl", head_dim=8)
    row = orc.index_maps(np.arange(L), L, p)["row"]
    assert row[10, 3] == 7 + L - 1 and row[3, 10] == -7 + L - 1


# ------------------------------------------------------------------------ brute force

@pytest.mark.parametrize("mech", orc.ALL_MECHS)
@pytest.mark.parametrize("mask", list(MASKS))
def test_vectorised_matches_scalar_brute_force(mech, mask):
    """Pin: pure-Python per-pair loops at L <= 8 agree with the vectorised oracle to 1e-12."""
    c, p = _case(mech, L=8, d=4, B=1, H=2, window=MASKS[mask], span=3, nb=8, md=6,
                 bidir=(mask != "causal"))
    q, k, v, tab, _ = _f64(c)
    O, LSE = orc.forward(p, q, k, v, tab)
    tl = {n: t.tolist() for n, t in tab.items()}
    for h in range(2):
        Ob, Lb = brute.forward_head(p, q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), tl, h)
        np.testing.assert_allclose(O[0, h], np.array(Ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[0, h], np.array(Lb), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------ library routine

def _zero_tables(c):
    return {n: np.zeros_like(t, dtype=np.float64) for n, t in c["tables"].items()}


@pytest.mark.parametrize("mech", orc.ALL_MECHS)
@pytest.mark.parametrize("mask", list(MASKS))
def test_zero_tables_reduce_to_sdpa(mech, mask):
    """Pin: with every table zero the oracle is plain attention; forward and all three
    input gradients match torch's scaled_dot_product_attention + autograd in float64."""
    c, p = _case(mech, L=24, d=8, B=2, H=3, window=MASKS[mask], span=4, nb=8, md=16,
                 bidir=(mask != "causal"))
    q, k, v, _, do = _f64(c)
    tab = _zero_tables(c)
    O, LSE = orc.forward(p, q, k, v, tab)
    dq, dk, dv, _ = orc.backward(p, q, k, v, tab, do)
    L = q.shape[2]
    mask_b = torch.from_numpy(orc.allowed_mask(np.arange(L), L, p))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask_b,
                                                           scale=p.s())
    ref.backward(torch.from_numpy(do))
    np.testing.assert_allclose(O, ref.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("mask", list(MASKS))
def test_alibi_matches_sdpa_with_an_explicit_bias(mask):
    """Pin: ALiBi equals torch's scaled_dot_product_attention with the float mask
    -m_h |i - j| (and -inf outside the window), forward and autograd gradients of q, k, v and
    the slopes, in float64."""
    c, p = _case("alibi", L=24, d=8, B=2, H=3, window=MASKS[mask], bidir=(mask != "causal"),
                 table_std=0.5)
    q, k, v, tab, do = _f64(c)
    O, _ = orc.forward(p, q, k, v, tab)
    dq, dk, dv, g = orc.backward(p, q, k, v, tab, do)
    L = q.shape[2]
    i = torch.arange(L, dtype=torch.float64)
    dist = (i[:, None] - i[None, :]).abs()
    m = torch.from_numpy(tab["slopes"].copy()).requires_grad_(True)
    allowed = torch.from_numpy(orc.allowed_mask(np.arange(L), L, p))
    bias = -m[:, None, None] * dist[None]
    mask_f = torch.where(allowed[None], bias, torch.full_like(bias, -math.inf))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask_f[None],
                                                           scale=p.s())
    ref.backward(torch.from_numpy(do))
    np.testing.assert_allclose(O, ref.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["slopes"], m.grad.numpy(), rtol=0, atol=1e-10)


def test_txl_position_free_is_attention_on_q_plus_u():
    """Pin: T-XL with r = 0 is plain attention with queries q + u (library routine)."""
    c, p = _case("txl", L=16, d=8, B=1, H=2, table_std=0.5)
    q, k, v, tab, do = _f64(c)
    tab["r"][:] = 0.0
    O, _ = orc.forward(p, q, k, v, tab)
    qu = q + tab["u"][None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qu), torch.from_numpy(k), torch.from_numpy(v), scale=p.s())
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)


def test_t5_constant_bias_is_plain_attention():
    """Pin: a T5 bias constant over buckets shifts every logit of a row equally."""
    c, p = _case("t5", L=20, d=8, B=1, H=2, nb=8, md=10)
    q, k, v, tab, _ = _f64(c)
    tab["beta"][:] = 1.75
    O, LSE = orc.forward(p, q, k, v, tab)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=p.s())
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask", list(MASKS))
def test_lse_closed_form(mask):
    """Pin: with q = 0 and zero tables every allowed logit is 0, so LSE_i = ln(#allowed keys)."""
    c, p = _case("shaw", L=12, d=4, window=MASKS[mask])
    q, k, v, tab, _ = _f64(c)
    q[:] = 0.0
    _, LSE = orc.forward(p, q, k, v, _zero_tables(c))
    L = 12
    for i in range(L):
        cnt = sum(1 for j in range(L)
                  if (p.window_left < 0 or i - j <= p.window_left)
                  and (p.window_right < 0 or j - i <= p.window_right))
        assert abs(LSE[0, 0, i] - math.log(cnt)) < 1e-14


# ------------------------------------------------------------------------ finite differences

def _loss(p, q, k, v, tab, do):
    O, _ = orc.forward(p, q, k, v, tab)
    return float(np.sum(O * do))


@pytest.mark.parametrize("mech", orc.ALL_MECHS)
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_gradients_match_central_differences(mech, mask):
    """Pin: every gradient element (q, k, v and every table) against central differences
    of the forward pass in float64, h = 1e-6."""
    c, p = _case(mech, L=6, d=3, B=1, H=2, window=MASKS[mask], span=2, nb=6, md=5,
                 bidir=(mask != "causal"), table_std=0.6)
    q, k, v, tab, do = _f64(c)
    dq, dk, dv, g = orc.backward(p, q, k, v, tab, do)
    h = 1e-6
    targets = [("q", q, dq), ("k", k, dk), ("v", v, dv)]
    targets += [(n, tab[n], g[n]) for n in tab]
    for name, x, grad in targets:
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(p, q, k, v, tab, do)
            x[idx] = old - h
            lm = _loss(p, q, k, v, tab, do)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.max(np.abs(fd))))
        assert np.max(np.abs(fd - grad)) <= 1e-6 * scale, name


@pytest.mark.parametrize("mech", orc.ALL_MECHS)
@pytest.mark.parametrize("mask", ["none", "causal", "local"])
def test_dq_rows_matches_central_differences(mech, mask):
    """Pin: the per-row dQ (used at lengths where the full backward is too large) against
    central differences of the forward pass on the selected query rows, h = 1e-6."""
    c, p = _case(mech, L=7, d=3, B=1, H=2, window=MASKS[mask], span=2, nb=6, md=5,
                 bidir=(mask != "causal"), table_std=0.6)
    q, k, v, tab, do = _f64(c)
    rows = np.array([0, 3, 6])
    h_ = 1e-6
    for hh in range(2):
        got = orc.dq_rows(p, q, k, v, tab, do, 0, hh, rows)
        for a, i in enumerate(rows):
            for e in range(q.shape[-1]):
                old = q[0, hh, i, e]
                q[0, hh, i, e] = old + h_
                lp = _loss(p, q, k, v, tab, do)
                q[0, hh, i, e] = old - h_
                lm = _loss(p, q, k, v, tab, do)
                q[0, hh, i, e] = old
                fd = (lp - lm) / (2 * h_)
                assert abs(fd - got[a, e]) <= 1e-6 * max(1.0, abs(fd)), (hh, i, e)


@pytest.mark.parametrize("mech", orc.ALL_MECHS)
@pytest.mark.parametrize("mask", ["none", "causal", "local"])
def test_dq_rows_is_a_row_subset_of_the_full_backward(mech, mask):
    """Pin: on a longer case, dq_rows over scattered rows equals those rows of the full
    backward (itself pinned by central differences)."""
    c, p = _case(mech, L=40, d=8, B=1, H=2, window=MASKS[mask], span=5, nb=10, md=20,
                 bidir=(mask != "causal"), table_std=0.6)
    q, k, v, tab, do = _f64(c)
    rows = np.array([0, 1, 7, 19, 20, 38, 39])
    dq, _, _, _ = orc.backward_head(p, q, k, v, tab, do, 0, 1)
    got = orc.dq_rows(p, q, k, v, tab, do, 0, 1, rows)
    assert np.allclose(got, dq[rows], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------ invariants

@pytest.mark.parametrize("mech", orc.MECHS)
def test_softmax_gradient_sums_vanish(mech):
    """Pin: sum_j dS_ij = 0 exactly, hence sum_c dbeta[h,c] = 0, sum_c dw[c] = 0,
    sum_c dKr[c] = 0 and sum_delta dr_h[delta] = 0."""
    c, p = _case(mech, L=30, d=8, B=2, H=2, span=5, nb=10, md=20, table_std=0.5)
    q, k, v, tab, do = _f64(c)
    _, _, _, g = orc.backward(p, q, k, v, tab, do)
    if mech == "t5":
        assert np.max(np.abs(g["beta"].sum(axis=1))) < 1e-12
    if mech == "shaw":
        assert np.max(np.abs(g["w"].sum(axis=0))) < 1e-12
    if mech == "deberta":
        assert np.max(np.abs(g["kr"].sum(axis=0))) < 1e-12
        assert np.max(np.abs(g["qr"].sum(axis=0))) > 1e-6   # column sums of dS do not vanish
    if mech == "txl":
        assert np.max(np.abs(g["r"].sum(axis=1))) < 1e-12


def test_shaw_causal_future_rows_have_zero_gradient():
    """Pin: under a causal mask no pair has j > i, so dw rows k+1..2k are exactly 0."""
    c, p = _case("shaw", L=16, d=4, window=(-1, 0), span=4)
    q, k, v, tab, do = _f64(c)
    _, _, _, g = orc.backward(p, q, k, v, tab, do)
    assert np.all(g["w"][5:] == 0.0)
    assert np.max(np.abs(g["w"][:5])) > 0


@pytest.mark.parametrize("mech", ["t5", "shaw", "txl"])
def test_key_shift_invariance(mech):
    """Pin: adding a constant vector to every key shifts each row's logits by one constant
    (the relative terms do not involve k for these mechanisms), so O is unchanged."""
    c, p = _case(mech, L=20, d=6, B=1, H=2, table_std=0.5, nb=8, md=10)
    q, k, v, tab, _ = _f64(c)
    O1, _ = orc.forward(p, q, k, v, tab)
    O2, _ = orc.forward(p, q, k + np.linspace(-1, 2, 6), v, tab)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)


def test_deberta_is_not_key_shift_invariant():
    c, p = _case("deberta", L=20, d=6, table_std=0.5)
    q, k, v, tab, _ = _f64(c)
    O1, _ = orc.forward(p, q, k, v, tab)
    O2, _ = orc.forward(p, q, k + np.linspace(-1, 2, 6), v, tab)
    assert np.max(np.abs(O1 - O2)) > 1e-6


# ------------------------------------------------------------------------ cross-mechanism

def test_shaw_equals_txl_with_reversed_table():
    """Pin: Shaw with k >= L-1 equals bidirectional T-XL with u = v = 0 and
    r[delta + L - 1] = w[k - delta]; gradients map the same way."""
    L, d, kk = 9, 4, 10
    c, p = _case("shaw", L=L, d=d, B=1, H=2, span=kk, table_std=0.8)
    q, k, v, tab, do = _f64(c)
    w = tab["w"]
    pt = orc.Params(mech="txl", head_dim=d)
    deltas = np.arange(-(L - 1), L)
    r = np.stack([w[kk - deltas]] * 2)                    # [H, 2L-1, d]
    tx = {"r": r, "u": np.zeros((2, d)), "v": np.zeros((2, d))}
    O1, L1 = orc.forward(p, q, k, v, tab)
    O2, L2 = orc.forward(pt, q, k, v, tx)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-12)
    g1 = orc.backward(p, q, k, v, tab, do)
    g2 = orc.backward(pt, q, k, v, tx, do)
    for a, b in zip(g1[:3], g2[:3]):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    dr = g2[3]["r"].sum(axis=0)                            # r shared via stacking
    np.testing.assert_allclose(g1[3]["w"][kk - deltas], dr, rtol=0, atol=1e-12)


def test_deberta_c2p_equals_shaw_and_p2c_is_its_transpose():
    """Pin: DeBERTa with Qr = 0 equals Shaw under the same scale with w[k_s - delta] =
    Kr[delta + k_d]; and swapping (q, Kr) with (k, Qr) transposes the score matrix."""
    L, d, kd, ks = 9, 4, 10, 9
    c, p = _case("deberta", L=L, d=d, B=1, H=1, span=kd, table_std=0.8)
    q, k, v, tab, _ = _f64(c)
    s = p.s()
    tab0 = {"kr": tab["kr"].copy(), "qr": np.zeros_like(tab["qr"])}
    w = np.zeros((2 * ks + 1, d))
    for delta in range(-(L - 1), L):
        w[ks - delta] = tab0["kr"][delta + kd]
    ps = orc.Params(mech="shaw", head_dim=d, rel_span=ks, scale=s)
    O1, _ = orc.forward(p, q, k, v, tab0)
    O2, _ = orc.forward(ps, q, k, v, {"w": w})
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)
    rows = np.arange(L)
    S = orc.scores_rows(p, q[0, 0], k[0, 0], tab, 0, rows)
    St = orc.scores_rows(p, k[0, 0], q[0, 0], {"kr": tab["qr"], "qr": tab["kr"]}, 0, rows)
    np.testing.assert_allclose(S, St.T, rtol=0, atol=1e-12)


def test_bias_is_toeplitz_for_constant_rows():
    """Pin: with every query row equal (Shaw, T-XL) or every key row equal (DeBERTa p2c)
    the additive term depends on i - j only."""
    for mech in ("shaw", "txl", "deberta"):
        c, p = _case(mech, L=14, d=4, B=1, H=1, span=4, table_std=0.8)
        q, k, v, tab, _ = _f64(c)
        q[:] = q[:, :, :1, :]
        k[:] = k[:, :, :1, :]
        Bm = orc.bias_rows(p, q[0, 0], k[0, 0], tab, 0, np.arange(14))
        np.testing.assert_allclose(Bm[1:, 1:], Bm[:-1, :-1], rtol=0, atol=1e-14)


# ------------------------------------------------------------------------ projections

def test_projection_matches_scalar_loops():
    """Pin: the table projection and its gradients against pure-Python loops."""
    rng = np.random.default_rng(5)
    N, F, H, d = 5, 4, 3, 2
    X = rng.standard_normal((N, F))
    W = rng.standard_normal((F, H * d))
    G = rng.standard_normal((H, N, d))
    rel = prj.project(X, W, H, d)
    dX, dW = prj.project_backward(X, W, G)
    for h in range(H):
        for n in range(N):
            for c in range(d):
                ref = sum(X[n][f] * W[f][h * d + c] for f in range(F))
                assert abs(rel[h, n, c] - ref) < 1e-12
    for f in range(F):
        for col in range(H * d):
            ref = sum(X[n][f] * G[col // d][n][col % d] for n in range(N))
            assert abs(dW[f, col] - ref) < 1e-12
    for n in range(N):
        for f in range(F):
            ref = sum(G[h][n][c] * W[f][h * d + c] for h in range(H) for c in range(d))
            assert abs(dX[n, f] - ref) < 1e-12


def test_projection_gradients_match_central_differences():
    """Pin: dX and dW of loss = sum(rel * G) against central differences, h = 1e-6."""
    rng = np.random.default_rng(6)
    N, F, H, d = 4, 3, 2, 3
    X = rng.standard_normal((N, F))
    W = rng.standard_normal((F, H * d))
    G = rng.standard_normal((H, N, d))
    dX, dW = prj.project_backward(X, W, G)
    h_ = 1e-6
    for arr, grad in ((X, dX), (W, dW)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h_
            lp = float(np.sum(prj.project(X, W, H, d) * G))
            arr[idx] = old - h_
            lm = float(np.sum(prj.project(X, W, H, d) * G))
            arr[idx] = old
            assert abs((lp - lm) / (2 * h_) - grad[idx]) < 1e-7



# ------------------------------------------------------------------------ table sharing across heads

LAYOUTS = [("shaw", "per_head"), ("deberta", "per_head"), ("txl", "shared")]


@pytest.mark.parametrize("mech,layout", LAYOUTS)
@pytest.mark.parametrize("mask", list(MASKS))
def test_table_layouts_match_scalar_brute_force(mech, layout, mask):
    """Pin: with one relation table per head (Shaw, DeBERTa) or one table for every head
    (T-XL), the pure-Python per-pair loops at L = 8 agree with the vectorised oracle to 1e-12."""
    c = make_case(mech, 1, 3, 8, 4, dtype="fp32", window=MASKS[mask], seed=17, rel_span=3,
                  bidirectional=(mask != "causal"), table_std=0.7, rel_layout=layout)
    p = orc.Params(**c["params"])
    q, k, v, tab, _ = _f64(c)
    O, LSE = orc.forward(p, q, k, v, tab)
    tl = {n: t.tolist() for n, t in tab.items()}
    for h in range(3):
        Ob, Lb = brute.forward_head(p, q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), tl, h)
        np.testing.assert_allclose(O[0, h], np.array(Ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[0, h], np.array(Lb), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mech,layout", LAYOUTS)
def test_table_layout_gradients_match_central_differences(mech, layout):
    """Pin: every gradient element, per-head and shared relation tables included, against
    central differences of the forward pass in float64, h = 1e-6."""
    c = make_case(mech, 2, 2, 6, 3, dtype="fp32", window=(-1, -1), seed=19, rel_span=2,
                  table_std=0.6, rel_layout=layout)
    p = orc.Params(**c["params"])
    q, k, v, tab, do = _f64(c)
    _, _, _, g = orc.backward(p, q, k, v, tab, do)
    h = 1e-6
    for name in tab:
        x = tab[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(p, q, k, v, tab, do)
            x[idx] = old - h
            lm = _loss(p, q, k, v, tab, do)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.max(np.abs(fd))))
        assert g[name].shape == x.shape
        assert np.max(np.abs(fd - g[name])) <= 1e-6 * scale, name


@pytest.mark.parametrize("mech", ["shaw", "deberta", "txl"])
def test_per_head_tables_decompose_into_single_head_problems(mech):
    """Pin: head h of a problem with one table per head is the one-head problem on that head's
    slices with that head's table; a table shared by every head gives the same outputs as one
    copy per head, and its gradient is the sum of the per-head copies' gradients."""
    layout = "shared" if mech == "txl" else "per_head"
    c = make_case(mech, 2, 3, 24, 8, dtype="fp32", window=(-1, -1), seed=23, rel_span=4,
                  table_std=0.5, rel_layout=layout)
    p = orc.Params(**c["params"])
    q, k, v, tab, do = _f64(c)
    O, LSE = orc.forward(p, q, k, v, tab)
    dq, dk, dv, g = orc.backward(p, q, k, v, tab, do)
    rel = orc.REL_TABLE_NDIM
    if layout == "per_head":
        for h in range(3):
            sub = {n: (t[h] if n in rel else t[h:h + 1]) for n, t in tab.items()}
            sl = slice(h, h + 1)
            O1, L1 = orc.forward(p, q[:, sl], k[:, sl], v[:, sl], sub)
            dq1, dk1, dv1, g1 = orc.backward(p, q[:, sl], k[:, sl], v[:, sl], sub, do[:, sl])
            assert np.allclose(O1, O[:, sl], rtol=0, atol=1e-13)
            assert np.allclose(L1, LSE[:, sl], rtol=0, atol=1e-13)
            for a, b_ in ((dq1, dq[:, sl]), (dk1, dk[:, sl]), (dv1, dv[:, sl])):
                assert np.allclose(a, b_, rtol=0, atol=1e-13)
            for n in g1:
                ref = g[n][h] if n in rel else g[n][h:h + 1]
                assert np.allclose(g1[n], ref, rtol=0, atol=1e-13), n
    else:
        rep = dict(tab)
        rep["r"] = np.repeat(tab["r"][None], 3, axis=0)
        O2, L2 = orc.forward(p, q, k, v, rep)
        dq2, dk2, dv2, g2 = orc.backward(p, q, k, v, rep, do)
        assert np.allclose(O2, O, rtol=0, atol=1e-13) and np.allclose(L2, LSE, rtol=0, atol=1e-13)
        for a, b_ in ((dq2, dq), (dk2, dk), (dv2, dv)):
            assert np.allclose(a, b_, rtol=0, atol=1e-13)
        assert np.allclose(g2["r"].sum(axis=0), g["r"], rtol=0, atol=1e-12)
        for n in ("u", "v"):
            assert np.allclose(g2[n], g[n], rtol=0, atol=1e-13)


# ------------------------------------------------------------------------ long-sequence backward

@pytest.mark.parametrize("mech", orc.ALL_MECHS)
@pytest.mark.parametrize("mask", ["none", "causal", "local"])
@pytest.mark.parametrize("chunk", [1, 7, 64])
def test_chunked_backward_equals_full_backward(mech, mask, chunk):
    """Pin: the query-row-chunked backward (used at 16K-32K tokens, where no L x L matrix fits)
    equals backward_head, itself pinned by central differences, to 1e-12, for chunk sizes that
    do and do not divide L, on every mechanism and mask (per-head tables for Shaw / DeBERTa,
    a shared T-XL table: both layouts of each go through the same code)."""
    for layout in (None, {"shaw": "per_head", "deberta": "per_head", "txl": "shared"}.get(mech)):
        c = make_case(mech, 1, 2, 45, 8, dtype="fp32", window=MASKS[mask], seed=37, rel_span=5,
                      num_buckets=10, max_distance=20, bidirectional=(mask != "causal"),
                      table_std=0.6, rel_layout=layout)
        p = orc.Params(**c["params"])
        q, k, v, tab, do = _f64(c)
        for hh in range(2):
            ref = orc.backward_head(p, q, k, v, tab, do, 0, hh)
            got = orc.backward_head_chunked(p, q, k, v, tab, do, 0, hh, chunk=chunk)
            for a, b_ in zip(got[:3], ref[:3]):
                assert np.allclose(a, b_, rtol=1e-12, atol=1e-12)
            assert set(got[3]) == set(ref[3])
            for n in ref[3]:
                assert np.allclose(got[3][n], ref[3][n], rtol=1e-12, atol=1e-12), n


@pytest.mark.parametrize("mech", orc.ALL_MECHS)
def test_chunk_forward_outputs_equal_forward_rows(mech):
    """Pin: the O and LSE rows that backward_chunk returns with its part equal forward_rows."""
    c, p = _case(mech, L=33, d=8, B=1, H=2, span=4, nb=8, md=16, table_std=0.6)
    q, k, v, tab, do = _f64(c)
    rows = np.array([0, 5, 6, 31, 32])
    part = orc.backward_chunk(p, q, k, v, tab, do, 0, 1, rows)
    O, lse = orc.forward_rows(p, q, k, v, tab, 0, 1, rows)
    assert np.array_equal(part["o"], O) and np.array_equal(part["lse"], lse)
