"""Shared helpers for the GPU parity tests: seeded cases, oracle runs and error metrics."""

from __future__ import annotations

import numpy as np

from exact_attention_relative_amd.inputs import make_case
from oracle import relpos_oracle as orc

# Tolerances stated for this path: bf16 inputs with fp32 accumulation -> O max-abs <= 1e-2 and
# relative L2 <= 2e-2 for every gradient; fp32 mode -> 1e-4 for both.
# LSE (derived, not stated): the denominator sums bf16-rounded weights, each within 2^-8 relative;
# fully correlated rounding (equal scores) moves ln of the sum by up to ln(1 + 2^-8) = 3.9e-3.
TOL = {"bf16": {"o": 1e-2, "grad": 2e-2, "lse": 4e-3},
       "fp32": {"o": 1e-4, "grad": 1e-4, "lse": 1e-4}}

MASKS = {"none": (-1, -1), "causal": (-1, 0), "local": (70, 45)}


def case(mech, B=2, H=3, L=200, dtype="bf16", mask="none", seed=7, span=None, table_std=None,
         nb=32, md=None, bidir=None, layout=None):
    window = MASKS[mask] if isinstance(mask, str) else mask
    if span is None:
        span = {"shaw": 48, "deberta": 40}.get(mech, 0)
    if md is None:
        md = max(16, L // 2)
    c = make_case(mech, B, H, L, 64, dtype=dtype, window=window, seed=seed, rel_span=span,
                  num_buckets=nb, max_distance=md, bidirectional=bidir, table_std=table_std,
                  rel_layout=layout)
    return c


def params(c) -> orc.Params:
    return orc.Params(**c["params"])


def tables64(c):
    return {n: t.astype(np.float64) for n, t in c["tables"].items()}


def oracle_forward(c):
    return orc.forward(params(c), c["q"], c["k"], c["v"], tables64(c))


def oracle_backward(c):
    return orc.backward(params(c), c["q"], c["k"], c["v"], tables64(c), c["dout"])


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b.ravel())
    num = np.linalg.norm((a - b).ravel())
    return num / den if den > 0 else num


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def halfulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 2.0 ** -133)


def check_row_sum_invariant(mech, case, o, tg):
    O = to_np(o)
    dO = case["dout"].astype(np.float64)
    q = case["q"].astype(np.float64)
    s = 1.0 / np.sqrt(3 * 64) if mech == "deberta" else 1.0 / 8.0
    # Each row of dS sums to dO_i . (O_i - O_i stored) because D is formed from the stored bf16
    # O; |that| <= e_i = sum_c |dO_ic| halfulp(O_ic), so the table gradients' sums over rows
    # are bounded by the matching weighted sums of e_i.
    e = np.sum(np.abs(dO) * halfulp_bf16(O), axis=-1)          # [B, H, L]
    slack = 1.25
    if mech == "t5":
        bound = e.sum(axis=(0, 2))                                # per head
        got = np.abs(tg["beta"].sum(axis=1))
        assert np.all(got <= slack * bound + 1e-4 * np.abs(tg["beta"]).max()), (got, bound)
    elif mech in ("shaw", "deberta"):
        name = "w" if mech == "shaw" else "kr"
        bound = s * np.einsum("bhl,bhld->d", e, np.abs(q))
        got = np.abs(tg[name].sum(axis=0))
        assert np.all(got <= slack * bound + 1e-4 * np.abs(tg[name]).max()), (got, bound)
    elif mech == "txl":
        v = case["tables"]["v"].astype(np.float64)
        bound = s * np.einsum("bhl,bhld->hd", e, np.abs(q + v[None, :, None, :]))
        got = np.abs(tg["r"].sum(axis=1))
        assert np.all(got <= slack * bound + 1e-4 * np.abs(tg["r"]).max()), (got.max(), bound.min())
