"""T-XL backward with its key-side r partials processed in groups of (batch, head) slices
(relpos_desc.max_partial_bytes): every gradient against the fp64 oracle for groups of one,
two and all six slices, with full span, causal and a two-sided window.  dQ, dK, dV, du and dv
do not depend on the grouping at all (bit for bit); dr only through the fixed order of its
fp32 sums, and a cap that fits every slice gives exactly the default result."""

import numpy as np
import pytest

from parity_util import MASKS, TOL, case, oracle_backward, rel_l2, to_np

pytestmark = pytest.mark.gpu


def _run(c, cap):
    import torch
    from exact_attention_relative_amd import runner
    desc = runner.desc_for(c)
    desc.max_partial_bytes = cap
    dev = runner.to_device(c)
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    torch.cuda.synchronize()
    return {k: v.clone() for k, v in g.items() if v is not None}


def _per_slice_bytes(L, window):
    nb = (L + 127) // 128
    rows = L + 256
    if window[0] >= 0 and window[1] >= 0:
        rows = min(rows, (window[0] + window[1] + 382 + 63) // 64 * 64)
    return nb * rows * 64 * 4


@pytest.mark.parametrize("mask", list(MASKS))
def test_txl_grouped_key_side_pass(mask):
    import torch
    L = 333
    c = case("txl", B=2, H=3, L=L, mask=mask, seed=91, table_std=0.5)
    window = MASKS[mask]
    per = _per_slice_bytes(L, window)
    print(f"txl groups mask={mask} per-slice={per}", flush=True)
    runs = {grp: _run(c, grp * per if grp else 0) for grp in (0, 1, 2, 6)}
    base = runs[0]
    # the grouping leaves every other output untouched
    for grp in (1, 2, 6):
        for name in ("dq", "dk", "dv", "dbias_a", "dbias_b"):
            assert torch.equal(runs[grp][name], base[name]), (grp, name)
    # a cap that holds all six slices is the default single group
    assert torch.equal(runs[6]["drel_a"], base["drel_a"])
    # every grouping matches the oracle's r gradient, and group sizes differ only by rounding
    _, _, _, tg = oracle_backward(c)
    tol = TOL["bf16"]["grad"]
    for grp in (1, 2, 6):
        err = rel_l2(to_np(runs[grp]["drel_a"]), tg["r"])
        assert err <= tol, (grp, err)
    np.testing.assert_allclose(to_np(runs[1]["drel_a"]), to_np(base["drel_a"]), rtol=1e-4,
                               atol=1e-6 * float(np.abs(to_np(base["drel_a"])).max()))
    # and each grouping is deterministic
    again = _run(c, per)
    assert torch.equal(again["drel_a"], runs[1]["drel_a"])
