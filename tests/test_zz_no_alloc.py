"""relpos_attn_fwd_noalloc (the forward for callers that cannot allocate) against
relpos_attn_fwd: two calls in a row through the C ABI, the second on a smaller problem, each
bitwise equal to the allocating entry point's O and LSE (the same kernels run on the same
inputs), for every mechanism."""

import numpy as np
import pytest

from parity_util import case, to_np

pytestmark = pytest.mark.gpu


def _noalloc(desc, dev, c):
    import torch
    from exact_attention_relative_amd import relpos_attn_fwd_noalloc, runner
    q = dev["q"]
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=q.device)
    relpos_attn_fwd_noalloc(desc, q, dev["k"], dev["v"], *runner.slots(dev), o, lse)
    return o, lse


@pytest.mark.parametrize("mech", ["t5", "shaw", "txl", "deberta", "alibi"])
def test_noalloc_forward_matches_allocating_forward_twice(mech):
    import torch
    from exact_attention_relative_amd import runner
    for i, (B, H, L, mask) in enumerate(((2, 4, 700, "none"), (1, 2, 150, "causal"))):
        c = case(mech, B=B, H=H, L=L, mask=mask, seed=97 + i, table_std=0.5)
        print(f"noalloc {mech} call {i} B={B} H={H} L={L}", flush=True)
        desc = runner.desc_for(c)
        dev = runner.to_device(c)
        o_ref, lse_ref = runner.forward(desc, dev)
        o, lse = _noalloc(desc, dev, c)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), (mech, i)
        assert torch.equal(lse, lse_ref), (mech, i)


def test_noalloc_refuses_a_workspace_beyond_the_scratch_array():
    import ctypes
    from exact_attention_relative_amd import (NOALLOC_SCRATCH_BYTES, RELPOS_E_WORKSPACE, load_library,
                                              make_desc, relpos_attn_workspace_size)
    desc = make_desc("deberta", 64, 16, 8192, rel_span=64)
    assert relpos_attn_workspace_size(desc, 0) > NOALLOC_SCRATCH_BYTES
    st = load_library().relpos_attn_fwd_noalloc(ctypes.byref(desc), None, None, None, None, None,
                                                None, None, None, None, None)
    assert st == RELPOS_E_WORKSPACE
