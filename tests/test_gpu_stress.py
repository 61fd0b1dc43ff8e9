"""Length stress: 16K and 32K tokens (B=1, H=2, d=64, bf16), every mechanism, bidirectional.

At these lengths the oracle's full backward (L x L matrices per slice) is too large, so the
GPU results are checked against what can be formed cheaply or holds at any size:

- O and LSE at sampled query rows (oracle forward rows);
- dQ at sampled query rows (oracle dq_rows, pinned by central differences);
- sum_j dV_j = sum_i dO_i (every softmax row sums to one), to the bf16 weight rounding;
- the table gradients' row-sum bound (each row of dS sums to the bf16 rounding of O);
- peak device memory below one fp32 [B, H, L, L] tensor.
"""

import numpy as np
import pytest

from parity_util import TOL, check_row_sum_invariant, rel_l2, to_np
from oracle import relpos_oracle as orc

pytestmark = pytest.mark.gpu

SETTINGS = {"t5": dict(num_buckets=32, max_distance=1024), "shaw": dict(rel_span=256),
            "deberta": dict(rel_span=512), "txl": {}, "alibi": {}}


def _case(mech, L):
    from exact_attention_relative_amd.inputs import make_case
    return make_case(mech, 1, 2, L, 64, dtype="bf16", window=(-1, -1), seed=L + 3,
                     sub=orc.ALL_MECHS.index(mech), **SETTINGS[mech])


def _rows(L):
    return np.unique(np.concatenate([np.linspace(0, L - 1, 12).astype(np.int64),
                                     np.array([1, 127, 128, L // 2 + 1, L - 2])]))


@pytest.mark.parametrize("L", [16384, 32768])
@pytest.mark.parametrize("mech", ["t5", "shaw", "deberta", "txl", "alibi"])
def test_long_sequence(mech, L):
    import torch
    from exact_attention_relative_amd import runner
    c = _case(mech, L)
    print(f"stress {mech} L={L}", flush=True)
    desc = runner.desc_for(c)
    dev = runner.to_device(c)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    naive = 1 * 2 * L * L * 4
    assert peak < naive, (peak, naive)

    p = orc.Params(**c["params"])
    tab = {n: t.astype(np.float64) for n, t in c["tables"].items()}
    tol = TOL["bf16"]
    rows = _rows(L)
    for h in range(2):
        O_ref, lse_ref = orc.forward_rows(p, c["q"], c["k"], c["v"], tab, 0, h, rows)
        assert np.max(np.abs(to_np(o[0, h])[rows] - O_ref)) <= tol["o"]
        assert np.max(np.abs(to_np(lse[0, h])[rows] - lse_ref)) <= tol["lse"]
        dq_ref = orc.dq_rows(p, c["q"], c["k"], c["v"], tab, c["dout"], 0, h, rows)
        assert rel_l2(to_np(g["dq"][0, h])[rows], dq_ref) <= tol["grad"]
        # every softmax row sums to one, so the columns of dV sum to the columns of dO
        sum_dv = to_np(g["dv"][0, h]).sum(axis=0)
        sum_do = c["dout"][0, h].astype(np.float64).sum(axis=0)
        assert rel_l2(sum_dv, sum_do) <= tol["grad"]
    tg = {n: to_np(t) for n, t in runner.named_table_grads(p.mech, g).items()}
    for n, t in tg.items():
        assert np.all(np.isfinite(t)), n
    check_row_sum_invariant(mech, c, o, tg)
