"""GPU checks that tie independent HIP paths together, each also against the fp64 oracle:

- batch-size stability: slice (b, h) of a B = 4 run is bitwise the same slice run alone (B = 1);
- Shaw with k >= L - 1 is bidirectional T-XL with u = v = 0 and one shared table r[m] = w[2k - m]
  (r reversed), so O, LSE, dQ, dK, dV agree and dr is dw reversed;
- DeBERTa with Qr = 0 is Shaw with span k and w = (Kr[2k-1], Kr[2k-1], Kr[2k-2], ..., Kr[0]) at
  the same scale, so dKr[2k-1] = dw[0] + dw[1] and dKr[r] = dw[2k - r] otherwise;
- K = 0 probes: the content scores vanish and S is the relative term alone (T-XL's u . k too).
"""

import numpy as np
import pytest

from parity_util import TOL, case, oracle_backward, oracle_forward, rel_l2, to_np

pytestmark = pytest.mark.gpu

MECHS = ["t5", "shaw", "txl", "deberta", "alibi"]


def _run(c, **desc_overrides):
    import torch
    from exact_attention_relative_amd import runner
    desc = runner.desc_for(c, **desc_overrides)
    dev = runner.to_device(c)
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    torch.cuda.synchronize()
    out = {"o": to_np(o), "lse": to_np(lse), "dq": to_np(g["dq"]), "dk": to_np(g["dk"]),
           "dv": to_np(g["dv"])}
    for name, t in runner.named_table_grads(c["params"]["mech"], g).items():
        out["table_" + name] = to_np(t)
    return out


def _check_oracle(c, got):
    tol = TOL["bf16"]
    O, LSE = oracle_forward(c)
    assert np.max(np.abs(got["o"] - O)) <= tol["o"]
    fin = np.isfinite(LSE)
    assert np.max(np.abs(got["lse"][fin] - LSE[fin])) <= tol["lse"]
    dq, dk, dv, tg = oracle_backward(c)
    ref = {"dq": dq, "dk": dk, "dv": dv, **{"table_" + n: g for n, g in tg.items()}}
    for n, r in ref.items():
        assert rel_l2(got[n], r) <= tol["grad"], (n, rel_l2(got[n], r))


@pytest.mark.parametrize("mech", MECHS)
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_batch_size_stability(mech, mask):
    """The per-slice outputs of a slice do not depend on the other slices of the batch."""
    c4 = case(mech, B=4, H=2, L=300, mask=mask, seed=51, table_std=0.5)
    print(f"batch stability {mech} {mask}", flush=True)
    g4 = _run(c4)
    for b in (0, 2):
        c1 = dict(c4)
        for n in ("q", "k", "v", "dout"):
            c1[n] = np.ascontiguousarray(c4[n][b:b + 1])
        c1["shape"] = (1,) + tuple(c4["shape"][1:])
        g1 = _run(c1)
        for n in ("o", "lse", "dq", "dk", "dv"):
            assert np.array_equal(g1[n][0], g4[n][b]), (n, b)


def _shaw_txl_pair(L, k, mask):
    from exact_attention_relative_amd.inputs import make_case
    shaw = case("shaw", B=2, H=2, L=L, mask=mask, span=k, seed=61, table_std=1.0)
    w = shaw["tables"]["w"]                            # [2k + 1, 64]
    window = (shaw["params"]["window_left"], shaw["params"]["window_right"])
    txl = make_case("txl", 2, 2, L, 64, window=window, seed=61)
    for n in ("q", "k", "v", "dout"):
        txl[n] = shaw[n]
    # bidirectional T-XL rows m = i - j + L - 1 read w[k - (i - j)] = w[k + L - 1 - m]
    m = np.arange(2 * L - 1)
    txl["tables"] = {"r": np.ascontiguousarray(w[k + L - 1 - m]),
                     "u": np.zeros((2, 64), np.float32), "v": np.zeros((2, 64), np.float32)}
    return shaw, txl


@pytest.mark.parametrize("mask", ["none", (90, 40)])
def test_shaw_full_span_equals_txl_with_reversed_shared_table(mask):
    L = 260
    k = L - 1 + 5   # k >= L - 1: no offset is clipped
    shaw, txl = _shaw_txl_pair(L, k, mask)
    print(f"shaw == txl identity mask={mask}", flush=True)
    gs = _run(shaw)
    gt = _run(txl)          # r [2L - 1, 64] without a head axis: one table for every head
    _check_oracle(shaw, gs)
    _check_oracle(txl, gt)
    tol = TOL["bf16"]
    assert np.max(np.abs(gs["o"] - gt["o"])) <= tol["o"]
    for n in ("dq", "dk", "dv"):
        assert rel_l2(gs[n], gt[n]) <= tol["grad"], n
    m = np.arange(2 * L - 1)
    dw_from_dr = np.zeros_like(gs["table_w"])
    dw_from_dr[k + L - 1 - m] = gt["table_r"]
    assert rel_l2(gs["table_w"], dw_from_dr) <= tol["grad"]
    # rows that no offset reads stay exactly zero on the Shaw side
    used = np.zeros(2 * k + 1, bool)
    used[k + L - 1 - m] = True
    assert np.all(gs["table_w"][~used] == 0.0)


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_deberta_c2p_equals_shaw(mask):
    from exact_attention_relative_amd.inputs import make_case
    L, k = 300, 40
    deb = case("deberta", B=2, H=2, L=L, mask=mask, span=k, seed=71, table_std=1.0)
    deb["tables"]["qr"] = np.zeros_like(deb["tables"]["qr"])
    deb["params"]["scale"] = 0.125
    kr = deb["tables"]["kr"]
    shaw = make_case("shaw", 2, 2, L, 64, window=(deb["params"]["window_left"],
                                                   deb["params"]["window_right"]),
                     seed=71, rel_span=k)
    for n in ("q", "k", "v", "dout"):
        shaw[n] = deb[n]
    idx = np.clip(2 * k - np.arange(2 * k + 1), 0, 2 * k - 1)
    shaw["tables"] = {"w": np.ascontiguousarray(kr[idx])}
    print(f"deberta c2p == shaw mask={mask}", flush=True)
    gd = _run(deb, scale=0.125)
    gs = _run(shaw)
    _check_oracle(deb, gd)
    _check_oracle(shaw, gs)
    tol = TOL["bf16"]
    assert np.max(np.abs(gd["o"] - gs["o"])) <= tol["o"]
    for n in ("dq", "dk", "dv"):
        assert rel_l2(gd[n], gs[n]) <= tol["grad"], n
    dkr = np.zeros_like(gd["table_kr"])
    np.add.at(dkr, idx, gs["table_w"])
    assert rel_l2(gd["table_kr"], dkr) <= tol["grad"]


@pytest.mark.parametrize("mech", MECHS)
@pytest.mark.parametrize("mask", ["none", "causal", "local"])
def test_zero_keys_expose_the_relative_term(mech, mask):
    """K = 0: S_ij is the relative term alone, so every index and table row shows in O, LSE and
    the gradients (amplified tables)."""
    c = case(mech, B=2, H=2, L=280, mask=mask, seed=81, table_std=1.0)
    c["k"] = np.zeros_like(c["k"])
    if mech == "t5":
        c["tables"]["beta"] = c["tables"]["beta"] * np.float32(4.0)
    print(f"K=0 {mech} {mask}", flush=True)
    _check_oracle(c, _run(c))
