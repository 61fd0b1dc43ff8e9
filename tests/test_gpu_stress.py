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


def test_txl_32k_partials_processed_in_groups():
    """Four heads at L = 32768 need 8.6 GB of key-side r partials, over the default 8 GiB cap:
    the backward runs in two slice groups, its workspace and peak memory stay under the cap, and
    the results pass the same sampled checks."""
    import torch
    from exact_attention_relative_amd import runner, relpos_attn_workspace_size
    from exact_attention_relative_amd.inputs import make_case
    L, H = 32768, 4
    c = make_case("txl", 1, H, L, 64, dtype="bf16", window=(-1, -1), seed=L + 11,
                  sub=orc.ALL_MECHS.index("txl"))
    print(f"stress txl grouped L={L} H={H}", flush=True)
    desc = runner.desc_for(c)
    per_slice = (L // 128) * (L + 256) * 64 * 4
    assert H * per_slice > 8 << 30
    ws = relpos_attn_workspace_size(desc, 1)
    assert ws < 8 << 30 and ws >= 3 * per_slice
    dev = runner.to_device(c)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() - base < (8 << 30) + (1 << 30)
    p = orc.Params(**c["params"])
    tab = {n: t.astype(np.float64) for n, t in c["tables"].items()}
    tol = TOL["bf16"]
    rows = _rows(L)
    for h in (0, H - 1):
        O_ref, lse_ref = orc.forward_rows(p, c["q"], c["k"], c["v"], tab, 0, h, rows)
        assert np.max(np.abs(to_np(o[0, h])[rows] - O_ref)) <= tol["o"]
        dq_ref = orc.dq_rows(p, c["q"], c["k"], c["v"], tab, c["dout"], 0, h, rows)
        assert rel_l2(to_np(g["dq"][0, h])[rows], dq_ref) <= tol["grad"]
    tg = {n: to_np(t) for n, t in runner.named_table_grads("txl", g).items()}
    for n, t in tg.items():
        assert np.all(np.isfinite(t)), n
    check_row_sum_invariant("txl", c, o, tg)
