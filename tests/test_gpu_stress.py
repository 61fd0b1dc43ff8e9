"""Length stress: 16K and 32K tokens, every mechanism, bidirectional, bf16.

Every output is compared with the fp64 oracle: O and LSE at every row, dQ, dK and dV of every
compared slice, and every table gradient (per-head tables at the compared heads).  The oracle's
backward is formed query-row chunk by chunk (backward_chunk, pinned against backward_head on the
CPU) over a pool of worker processes (tests/oracle_pool.py).  16K runs two heads, 32K one (the
oracle takes about half a minute per 32K slice on 16 cores).  Also checked on the complete GPU
outputs: sum_j dV_j = sum_i dO_i, the table gradients' row-sum bound, and peak device memory
below one fp32 [B, H, L, L] tensor."""

import numpy as np
import pytest

from oracle_pool import oracle_long
from parity_util import TOL, check_row_sum_invariant, rel_l2, to_np
from oracle import relpos_oracle as orc

pytestmark = pytest.mark.gpu

SETTINGS = {"t5": dict(num_buckets=32, max_distance=1024), "shaw": dict(rel_span=256),
            "deberta": dict(rel_span=512), "txl": {}, "alibi": {}}
REL = ("w", "r", "kr", "qr")


def _case(mech, L, H):
    from exact_attention_relative_amd.inputs import make_case
    return make_case(mech, 1, H, L, 64, dtype="bf16", window=(-1, -1), seed=L + 3,
                     sub=orc.ALL_MECHS.index(mech), **SETTINGS[mech])


def _gpu(c):
    import torch
    from exact_attention_relative_amd import runner
    desc = runner.desc_for(c)
    dev = runner.to_device(c)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    return o, lse, g, peak


def _compare(c, o, lse, g, slices):
    """Every output of the slices in `slices` against the oracle; table gradients when the
    slices are every reader of the compared table rows."""
    from exact_attention_relative_amd import runner
    mech = c["params"]["mech"]
    tol = TOL["bf16"]
    ref = oracle_long(c, slices)
    for (b, h) in slices:
        O = to_np(o[b, h])
        assert np.max(np.abs(O - ref["o"][(b, h)])) <= tol["o"], (b, h)
        assert np.max(np.abs(to_np(lse[b, h]) - ref["lse"][(b, h)])) <= tol["lse"], (b, h)
        for n in ("dq", "dk", "dv"):
            e = rel_l2(to_np(g[n][b, h]), ref[n][(b, h)])
            assert e <= tol["grad"], (n, b, h, e)
    heads = sorted({h for _, h in slices})
    B, H = c["q"].shape[:2]
    all_slices = len(slices) == B * H
    tg = {n: to_np(t) for n, t in runner.named_table_grads(mech, g).items()}
    for n, got in tg.items():
        per_head = orc.has_head_axis(n, c["tables"][n])
        if not per_head and not all_slices:
            continue   # a shared table's gradient sums slices not compared here
        if per_head:
            got, want = got[heads], ref["g"][n][heads]
        else:
            want = ref["g"][n]
        e = rel_l2(got, want)
        assert e <= tol["grad"], (n, e)


@pytest.mark.parametrize("L,H", [(16384, 2), (32768, 1)])
@pytest.mark.parametrize("mech", ["t5", "shaw", "deberta", "txl", "alibi"])
def test_long_sequence(mech, L, H):
    c = _case(mech, L, H)
    print(f"stress {mech} L={L} H={H}", flush=True)
    o, lse, g, peak = _gpu(c)
    naive = 1 * H * L * L * 4
    assert peak < naive, (peak, naive)
    _compare(c, o, lse, g, [(0, h) for h in range(H)])
    # every softmax row sums to one, so the columns of dV sum to the columns of dO
    for h in range(H):
        sum_dv = to_np(g["dv"][0, h]).sum(axis=0)
        sum_do = c["dout"][0, h].astype(np.float64).sum(axis=0)
        assert rel_l2(sum_dv, sum_do) <= TOL["bf16"]["grad"]
    from exact_attention_relative_amd import runner
    tg = {n: to_np(t) for n, t in runner.named_table_grads(mech, g).items()}
    check_row_sum_invariant(mech, c, o, tg)


def test_txl_32k_partials_processed_in_groups():
    """Four heads at L = 32768 would need 8.6 GB of key-side r partials at once: with 256 key
    blocks per slice the default groups hold two slices (512 workgroups), so the backward runs
    in two slice groups with about 4.3 GB of partials, and heads 0 and 3 (one in each group)
    match the oracle in every output, their r, u and v gradients included."""
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
    assert 2 * per_slice <= ws < 3 * per_slice
    o, lse, g, peak = _gpu(c)
    assert peak < 3 * per_slice + (1 << 30)
    _compare(c, o, lse, g, [(0, 0), (0, H - 1)])
    tg = {n: to_np(t) for n, t in runner.named_table_grads("txl", g).items()}
    check_row_sum_invariant("txl", c, o, tg)
