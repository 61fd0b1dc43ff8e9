"""Local (sliding-window) attention at L = 8192: the tile scheduler visits only the key tiles
inside each block's window, so a window of w keys costs about w / L of the full sweep.

Every output is checked against the fp64 oracle's full backward of the slice (B = 1, H = 1):
O and LSE, dQ, dK, dV and the table gradients, for a symmetric window of 256 and a causal
window of 512 (T5 then uses its unidirectional bucket map)."""

import numpy as np
import pytest

from parity_util import TOL, rel_l2, to_np
from oracle import relpos_oracle as orc

pytestmark = pytest.mark.gpu

SETTINGS = {"t5": dict(num_buckets=32, max_distance=1024), "shaw": dict(rel_span=256),
            "deberta": dict(rel_span=512), "txl": {}, "alibi": {}}


@pytest.mark.parametrize("window", [(256, 256), (512, 0)])
@pytest.mark.parametrize("mech", ["t5", "shaw", "deberta", "txl", "alibi"])
def test_local_window_L8192(mech, window):
    import torch
    from exact_attention_relative_amd import runner
    from exact_attention_relative_amd.inputs import make_case
    c = make_case(mech, 1, 1, 8192, 64, dtype="bf16", window=window, seed=17,
                  sub=orc.ALL_MECHS.index(mech), **SETTINGS[mech])
    print(f"local {mech} window={window}", flush=True)
    desc = runner.desc_for(c)
    dev = runner.to_device(c)
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    torch.cuda.synchronize()

    p = orc.Params(**c["params"])
    tab = {n: t.astype(np.float64) for n, t in c["tables"].items()}
    tol = TOL["bf16"]
    O_ref, lse_ref = orc.forward_rows(p, c["q"], c["k"], c["v"], tab, 0, 0)
    assert np.max(np.abs(to_np(o[0, 0]) - O_ref)) <= tol["o"]
    assert np.max(np.abs(to_np(lse[0, 0]) - lse_ref)) <= tol["lse"]
    dq, dk, dv, gref = orc.backward_head(p, c["q"], c["k"], c["v"], tab, c["dout"], 0, 0)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert rel_l2(to_np(g[name][0, 0]), ref) <= tol["grad"], name
    got = {n: to_np(t) for n, t in runner.named_table_grads(p.mech, g).items()}
    for n, ref in gref.items():
        t = got[n][0] if n in ("beta", "r", "u", "v") else got[n]
        assert rel_l2(t, ref) <= tol["grad"], (n, rel_l2(t, ref))
