"""GPU parity of the forward pass (O, LSE) and of the index maps against the fp64 oracle."""

import numpy as np
import pytest

from parity_util import MASKS, TOL, case, oracle_forward, params, to_np
from oracle import relpos_oracle as orc

pytestmark = pytest.mark.gpu

MECHS = ["t5", "shaw", "txl", "deberta", "alibi"]


def _run_fwd(c):
    from exact_attention_relative_amd import runner
    desc = runner.desc_for(c)
    dev = runner.to_device(c)
    o, lse = runner.forward(desc, dev)
    import torch
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


def _check_fwd(c, o, lse):
    O, LSE = oracle_forward(c)
    tol = TOL[c["dtype"]]
    assert np.max(np.abs(O)) < 4.0  # bf16 output rounding stays below the tolerance
    err_o = np.max(np.abs(o - O))
    fin = np.isfinite(LSE)
    assert np.array_equal(np.isfinite(lse), fin)
    err_l = np.max(np.abs(lse[fin] - LSE[fin])) if fin.any() else 0.0
    assert err_o <= tol["o"], f"O max-abs {err_o}"
    assert err_l <= tol["lse"], f"LSE max-abs {err_l}"
    return err_o, err_l


@pytest.mark.parametrize("mech", MECHS)
@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("L", [200, 333])
def test_forward_bf16(mech, mask, L):
    """Several 128-row blocks, 64-key tiles and a ragged tail, every mask."""
    c = case(mech, B=2, H=3, L=L, mask=mask, seed=L + len(mask))
    print(f"fwd bf16 mech={mech} mask={mask} L={L}", flush=True)
    o, lse = _run_fwd(c)
    _check_fwd(c, o, lse)


@pytest.mark.parametrize("mech", MECHS)
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_forward_bf16_amplified_tables(mech, mask):
    """Relative terms with unit-scale tables so an indexing slip moves O well past tolerance."""
    c = case(mech, B=1, H=2, L=300, mask=mask, table_std=1.0, seed=3)
    if mech == "t5":
        c["tables"]["beta"] = c["tables"]["beta"] * np.float32(4.0)
    o, lse = _run_fwd(c)
    _check_fwd(c, o, lse)


@pytest.mark.parametrize("mech", MECHS)
@pytest.mark.parametrize("mask", ["none", "causal", "local"])
def test_forward_fp32(mech, mask):
    c = case(mech, B=1, H=2, L=190, dtype="fp32", mask=mask, seed=11, table_std=0.5)
    o, lse = _run_fwd(c)
    _check_fwd(c, o, lse)


def test_forward_t5_fp32_reference_config():
    """T5 bucketed bias, fp32, B=1 H=1 L=128 d=64, 32 buckets, max_distance 128, seed 0."""
    from exact_attention_relative_amd.inputs import make_config
    c = make_config("t5_fp32_L128")
    o, lse = _run_fwd(c)
    _check_fwd(c, o, lse)


@pytest.mark.parametrize("mech", MECHS)
def test_forward_small_spans_and_short_sequences(mech):
    """Spans shorter than one tile, sequences shorter than one tile."""
    for L, span in [(1, 1), (5, 1), (37, 2), (64, 3), (129, 7)]:
        c = case(mech, B=1, H=2, L=L, span=span, md=max(4, L), nb=8, seed=L)
        o, lse = _run_fwd(c)
        _check_fwd(c, o, lse)


def test_forward_empty_is_noop():
    import torch
    from exact_attention_relative_amd import make_desc, relpos_attn_fwd
    for B, L in [(0, 64), (2, 0)]:
        desc = make_desc("shaw", B, 2, L, rel_span=4)
        q = torch.empty((max(B, 1), 2, max(L, 1), 64), dtype=torch.bfloat16, device="cuda")
        w = torch.zeros((9, 64), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((1,), dtype=torch.float32, device="cuda")
        assert relpos_attn_fwd(desc, q, q, q, w, None, None, None, q, lse, None, 0) == 0


@pytest.mark.parametrize("mech", MECHS)
def test_forward_deterministic(mech):
    c = case(mech, B=1, H=2, L=260, seed=5)
    o1, l1 = _run_fwd(c)
    o2, l2 = _run_fwd(c)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("mech,mask,extra", [
    ("t5", "none", dict(nb=32, md=128)), ("t5", "causal", dict(nb=32, md=1024)),
    ("t5", "none", dict(nb=32, md=1024)), ("t5", "none", dict(nb=16, md=40)),
    ("shaw", "none", {}), ("shaw", "causal", {}), ("txl", "none", {}), ("txl", "causal", {}),
    ("deberta", "none", {}), ("deberta", "local", {}), ("alibi", "none", {}), ("alibi", "causal", {})])
def test_index_maps_bit_exact(mech, mask, extra):
    """Bucket / clamp rows of every offset |i - j| < L, computed by the library on the GPU."""
    import torch
    from exact_attention_relative_amd import relpos_index_map, runner
    L = 2500
    c = case(mech, B=1, H=1, L=L, mask=mask, **extra)
    desc = runner.desc_for(c)
    a = torch.full((2 * L - 1,), -7, dtype=torch.int32, device="cuda")
    b = torch.full((2 * L - 1,), -7, dtype=torch.int32, device="cuda") if mech == "deberta" else None
    relpos_index_map(desc, a, b)
    torch.cuda.synchronize()
    p = params(c)
    # oracle: row of offset delta = i - j read off its pair index maps at i = L - 1 and i = 0
    deltas = np.arange(-(L - 1), L)
    rows_i = np.where(deltas >= 0, deltas, 0)
    cols_j = rows_i - deltas
    maps = orc.index_maps(np.arange(L), L, p)
    key = {"t5": "bucket", "shaw": "row", "txl": "row", "deberta": "c2p", "alibi": "dist"}[mech]
    exp_a = maps[key][rows_i, cols_j]
    if mech == "txl":
        nrel = orc.txl_rows(L, p)
        exp_a = np.where((exp_a >= 0) & (exp_a < nrel), exp_a, -1)
    assert np.array_equal(a.cpu().numpy(), exp_a)
    if mech == "deberta":
        assert np.array_equal(b.cpu().numpy(), maps["p2c"][rows_i, cols_j])
