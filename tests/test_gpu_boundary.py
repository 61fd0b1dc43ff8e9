"""GPU checks of the C-ABI boundary: relation tables per head or shared by every head
(rel_head_stride), and calls with no pairs (L = 0 or B = 0), which must still overwrite every
table gradient with zeros."""

import numpy as np
import pytest

from parity_util import MASKS, TOL, case, oracle_backward, oracle_forward, rel_l2, to_np

pytestmark = pytest.mark.gpu

# non-default layouts: Shaw / DeBERTa one table per head, T-XL one table for every head
LAYOUTS = [("shaw", "per_head"), ("deberta", "per_head"), ("txl", "shared")]


def _run(c):
    import torch
    from exact_attention_relative_amd import runner
    desc = runner.desc_for(c)
    dev = runner.to_device(c)
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    torch.cuda.synchronize()
    out = {"o": to_np(o), "lse": to_np(lse), "dq": to_np(g["dq"]), "dk": to_np(g["dk"]),
           "dv": to_np(g["dv"])}
    for name, t in runner.named_table_grads(c["params"]["mech"], g).items():
        out["table_" + name] = to_np(t)
    return desc, out


@pytest.mark.parametrize("mech,layout", LAYOUTS)
@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("std", [None, 1.0])
def test_table_layouts_match_oracle(mech, layout, mask, std):
    c = case(mech, B=2, H=3, L=333, mask=mask, seed=41 + len(mask), table_std=std, layout=layout)
    print(f"layout {mech} {layout} mask={mask} std={std}", flush=True)
    desc, got = _run(c)
    expect_stride = 0 if layout == "shared" else int(np.prod(c["tables"][
        "w" if mech == "shaw" else "kr"].shape[1:]))
    assert desc.rel_head_stride == expect_stride
    tol = TOL["bf16"]
    O, LSE = oracle_forward(c)
    assert np.max(np.abs(got["o"] - O)) <= tol["o"]
    assert np.max(np.abs(got["lse"] - LSE)) <= tol["lse"]
    dq, dk, dv, tg = oracle_backward(c)
    ref = {"dq": dq, "dk": dk, "dv": dv}
    ref.update({"table_" + n: g for n, g in tg.items()})
    for n, r in ref.items():
        assert got[n].shape == r.shape, n
        assert rel_l2(got[n], r) <= tol["grad"], (n, rel_l2(got[n], r))


@pytest.mark.parametrize("mech", ["t5", "shaw", "txl", "deberta", "alibi"])
@pytest.mark.parametrize("B,L", [(2, 0), (0, 64)])
@pytest.mark.parametrize("per_head", [False, True])
def test_no_pairs_overwrites_table_grads_with_zeros(mech, B, L, per_head):
    """Every table gradient is overwritten: with no pairs it must come back zero, whatever the
    buffer held before (here 7.0)."""
    import torch
    from exact_attention_relative_amd import make_desc, relpos_attn_bwd, relpos_attn_workspace_size
    H, k = 3, 4
    # table rows (the bidirectional T-XL table has 2L - 1 rows: none when L = 0)
    rows = {"shaw": 2 * k + 1, "deberta": 2 * k, "txl": max(2 * L - 1, 0)}.get(mech, 0)
    stride = rows * 64 if (per_head and rows) else 0
    desc = make_desc(mech, B, H, L, rel_span=k, num_buckets=8, max_distance=16,
                     rel_head_stride=stride)
    dt, dev = torch.bfloat16, "cuda"
    q = torch.zeros((max(B, 1), H, max(L, 1), 64), dtype=dt, device=dev)
    lse = torch.zeros((max(B, 1), H, max(L, 1)), dtype=torch.float32, device=dev)
    ntab = H if stride else 1
    tabs = {"rel_a": None, "rel_b": None, "bias_a": None, "bias_b": None}
    if mech in ("shaw", "deberta", "txl"):
        shape = (ntab, max(rows, 1), 64)
        tabs["rel_a"] = torch.zeros(shape, dtype=dt, device=dev)
        if mech == "deberta":
            tabs["rel_b"] = torch.zeros(shape, dtype=dt, device=dev)
    if mech == "t5":
        tabs["bias_a"] = torch.zeros((H, 8), dtype=torch.float32, device=dev)
    if mech == "alibi":
        tabs["bias_a"] = torch.zeros((H,), dtype=torch.float32, device=dev)
    if mech == "txl":
        tabs["bias_a"] = torch.zeros((H, 64), dtype=torch.float32, device=dev)
        tabs["bias_b"] = torch.zeros((H, 64), dtype=torch.float32, device=dev)
    grads = {n: (None if t is None else torch.full(t.shape, 7.0, dtype=torch.float32, device=dev))
             for n, t in tabs.items()}
    n_ws = relpos_attn_workspace_size(desc, 1)
    ws = torch.empty(max(n_ws, 256), dtype=torch.uint8, device=dev)
    relpos_attn_bwd(desc, q, q, q, q, lse, q, tabs["rel_a"], tabs["rel_b"], tabs["bias_a"],
                    tabs["bias_b"], q, q, q, grads["rel_a"], grads["rel_b"], grads["bias_a"],
                    grads["bias_b"], ws, n_ws)
    torch.cuda.synchronize()
    print(f"no pairs {mech} B={B} L={L} per_head={per_head}", flush=True)
    for n, g in grads.items():
        if g is None:
            continue
        # the gradient region the call owns: `rows` rows per table for the relation tables
        written = (g[:, :rows] if n in ("rel_a", "rel_b") else g).reshape(-1)
        if written.numel():
            assert float(written.abs().max()) == 0.0, n
