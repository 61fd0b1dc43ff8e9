"""GPU parity of the folded passes.

Once the batch entries of a head fill a wave of workgroups, the general passes of Shaw and DeBERTa
and the T-XL key-side pass run the batch entries as consecutive launches into one set of
partials: the first launch stores each partial element, every later one adds to it.  At B = 3,
H = 16, L = 2048 (256 workgroups per batch entry) per-head tables fold the batch entries in two
groups, {0, 1} and {2}, so the second launch skips the workgroups of the short group; tables
shared by every head fold whole (batch, head) slices, here in pairs.  Checked on every output against the fp64
oracle (all slices, all rows, every table gradient), for shared and per-head tables, in bf16 and
fp32, and run twice for bitwise determinism."""

import numpy as np
import pytest

from oracle_pool import oracle_long
from parity_util import TOL, case, rel_l2, to_np

pytestmark = pytest.mark.gpu

B, H, L = 3, 16, 2048


def _gpu(c):
    import torch
    from exact_attention_relative_amd import runner
    desc = runner.desc_for(c)
    dev = runner.to_device(c)
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    torch.cuda.synchronize()
    out = {"o": to_np(o), "lse": to_np(lse), "dq": to_np(g["dq"]), "dk": to_np(g["dk"]),
           "dv": to_np(g["dv"])}
    for n, t in runner.named_table_grads(c["params"]["mech"], g).items():
        out["table_" + n] = to_np(t)
    return out


def _folds(mech, span):
    """The folding is on at B = 3: one more batch entry adds no partial slots there (B = 2 and
    B = 3 both hold two groups), while going from B = 1 to B = 2 adds a group."""
    import exact_attention_relative_amd as ear
    ws = {b: ear.relpos_attn_workspace_size(ear.make_desc(mech, b, H, L, rel_span=span), 1)
          for b in (1, 2, 3)}
    return ws[3] - ws[2] < ws[2] - ws[1]


@pytest.mark.parametrize("mech,span,layout,dtype", [
    ("shaw", 300, None, "bf16"), ("deberta", 200, None, "bf16"),
    ("shaw", 100, "per_head", "bf16"), ("deberta", 64, "per_head", "bf16"),
    ("deberta", 160, None, "fp32"), ("txl", 0, None, "bf16"), ("txl", 0, "shared", "bf16"),
    ("txl", 0, None, "fp32")])
def test_folded_general_passes(mech, span, layout, dtype):
    assert _folds(mech, span)
    c = case(mech, B=B, H=H, L=L, span=span, layout=layout, dtype=dtype, seed=span + 3)
    print(f"folded {mech} span={span} layout={layout} {dtype}", flush=True)
    got = _gpu(c)
    again = _gpu(c)
    for k in got:
        assert np.array_equal(got[k], again[k]), k
    ref = oracle_long(c, [(b, h) for b in range(B) for h in range(H)])
    tol = TOL[dtype]
    stack = lambda d: np.stack([np.stack([d[(b, h)] for h in range(H)]) for b in range(B)])
    assert np.max(np.abs(got["o"] - stack(ref["o"]))) <= tol["o"]
    assert np.max(np.abs(got["lse"] - stack(ref["lse"]))) <= tol["lse"]
    for key in ("dq", "dk", "dv"):
        e = rel_l2(got[key], stack(ref[key]))
        print(f"  {key} rel-L2 {e:.2e}", flush=True)
        assert e <= tol["grad"], key
    for n, t in ref["g"].items():
        e = rel_l2(got["table_" + n], t)
        print(f"  table {n} rel-L2 {e:.2e}", flush=True)
        assert e <= tol["grad"], n
