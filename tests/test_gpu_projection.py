"""Relation-table projections on the GPU against the fp64 oracle (oracle/projection.py).

rel = X W (head-split to [H, N, d]) and its gradients dX = dY W^T, dW = X^T dY.  Error bounds
follow from the arithmetic, element by element, with A = the same products over |X|, |W|,
|drel| (the oracle on absolute values):

- bf16 tables: the fp32-accumulated sum (error <= 2^-14 A for F <= 1024) is rounded once to
  bf16 (<= 2^-8 of the value), so |got - ref| <= 2^-8 |ref| + 2^-13 A;
- fp32 results: operands split into two bf16 parts drop lo x lo (and leave 2^-18 of each
  operand), about 2^-16 A, plus fp32 accumulation: |got - ref| <= 1e-4 A.

Shapes: a ragged one (N, F, H d not multiples of the 64-wide tiles, d = 40 splitting heads
inside a tile); the DeBERTa bases of spans 256 and 512 (2k rows of width d = 64, with W_r^k and
W_r^q side by side as two heads, so one call gives Kr and Qr); the T-XL bases of L = 8192
(sinusoid features of width 512, 8 heads of 64), causal (8192 offsets) and full-span (16383);
a long basis reduced over many dW slices; and a single row."""

import numpy as np
import pytest

from parity_util import TOL, rel_l2, to_np
from oracle import projection as prj

pytestmark = pytest.mark.gpu

SHAPES = {
    "ragged": ((300, 136, 3, 40), "normal", None),
    "deberta_span256": ((512, 64, 2, 64), "normal", None),
    "deberta_span512": ((1024, 64, 2, 64), "normal", None),
    "txl_L8192_causal": ((8192, 512, 8, 64), "sinusoid", 0),
    "txl_L8192_full": ((16383, 512, 8, 64), "sinusoid", None),
    "long_slices": ((5000, 64, 1, 64), "normal", None),
    "one_row": ((1, 8, 1, 8), "normal", None),
}


def _case(name, dtype, seed=5):
    from exact_attention_relative_amd.inputs import make_projection_case
    (N, F, H, d), basis, first = SHAPES[name]
    return make_projection_case(N, F, H, d, dtype=dtype, basis=basis, first_offset=first,
                                seed=seed, sub=list(SHAPES).index(name))


def _dev(c):
    from exact_attention_relative_amd.runner import tensor_from_f32
    return (tensor_from_f32(c["X"], c["dtype"]), tensor_from_f32(c["W"], c["dtype"]),
            tensor_from_f32(c["drel"], "fp32"))


def _desc(c):
    import exact_attention_relative_amd as ear
    N, F, H, d = c["shape"]
    return ear.make_proj_desc(N, F, H, d, dtype=c["dtype"])


def _run_bwd(c, X, W, drel, want_dx=True, want_dw=True):
    import torch
    import exact_attention_relative_amd as ear
    N, F, H, d = c["shape"]
    desc = _desc(c)
    dX = torch.full((N, F), float("nan"), device="cuda") if want_dx else None
    dW = torch.full((F, H * d), float("nan"), device="cuda") if want_dw else None
    n = ear.relpos_project_workspace_size(desc)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    ear.relpos_project_bwd(desc, X, W, drel, dX, dW, ws, n)
    return dX, dW


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("name", list(SHAPES))
def test_project_forward(name, dtype):
    import torch
    import exact_attention_relative_amd as ear
    c = _case(name, dtype)
    N, F, H, d = c["shape"]
    print(f"project fwd {name} {dtype} {c['shape']}", flush=True)
    X, W, _ = _dev(c)
    rel = torch.full((H, N, d), float("nan"), device="cuda",
                     dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    ear.relpos_project_fwd(_desc(c), X, W, rel)
    torch.cuda.synchronize()
    got = to_np(rel)
    ref = prj.project(c["X"], c["W"], H, d)
    A = prj.project(np.abs(c["X"]), np.abs(c["W"]), H, d)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -13 * A if dtype == "bf16" else 1e-4 * A
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) - bound)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("name", list(SHAPES))
def test_project_backward(name, dtype):
    import torch
    c = _case(name, dtype)
    print(f"project bwd {name} {dtype} {c['shape']}", flush=True)
    X, W, drel = _dev(c)
    dX, dW = _run_bwd(c, X, W, drel)
    torch.cuda.synchronize()
    dX_ref, dW_ref = prj.project_backward(c["X"], c["W"], c["drel"])
    AX, AW = prj.project_backward(np.abs(c["X"]), np.abs(c["W"]), np.abs(c["drel"]))
    for got, ref, A in ((to_np(dX), dX_ref, AX), (to_np(dW), dW_ref, AW)):
        assert np.all(np.isfinite(got))
        assert np.all(np.abs(got - ref) <= 1e-4 * A), np.max(np.abs(got - ref) - 1e-4 * A)


def test_project_backward_is_deterministic_and_grads_are_independent():
    """Repeated calls agree bit for bit; asking for dW alone or dX alone gives the same bits."""
    import torch
    c = _case("txl_L8192_full", "bf16")
    X, W, drel = _dev(c)
    dX1, dW1 = _run_bwd(c, X, W, drel)
    dX2, dW2 = _run_bwd(c, X, W, drel)
    _, dW3 = _run_bwd(c, X, W, drel, want_dx=False)
    dX4, _ = _run_bwd(c, X, W, drel, want_dw=False)
    torch.cuda.synchronize()
    assert torch.equal(dX1, dX2) and torch.equal(dW1, dW2)
    assert torch.equal(dW1, dW3) and torch.equal(dX1, dX4)


def test_empty_basis_gives_zero_weight_gradient():
    import torch
    import exact_attention_relative_amd as ear
    from exact_attention_relative_amd.inputs import make_projection_case
    c = make_projection_case(0, 64, 2, 32, dtype="bf16")
    X = torch.empty((1, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((64, 64), dtype=torch.bfloat16, device="cuda")
    drel = torch.empty((2, 1, 32), device="cuda")
    dW = torch.full((64, 64), float("nan"), device="cuda")
    desc = ear.make_proj_desc(0, 64, 2, 32)
    assert ear.relpos_project_workspace_size(desc) == 0
    ear.relpos_project_bwd(desc, X, W, drel, None, dW, None, 0)
    torch.cuda.synchronize()
    assert c["X"].shape == (0, 64)
    assert torch.count_nonzero(dW).item() == 0


def test_txl_projection_chained_with_attention():
    """r = R W_r on the GPU feeds the T-XL attention; its table gradient feeds dW_r.  Checked
    against the oracle's projection and full backward at L = 256, B = 1, H = 2."""
    import torch
    import exact_attention_relative_amd as ear
    from exact_attention_relative_amd import runner
    from exact_attention_relative_amd.inputs import make_case, make_projection_case
    from oracle import relpos_oracle as orc
    L, H, d, F = 256, 2, 64, 128
    c = make_case("txl", 1, H, L, d, dtype="bf16", seed=23, table_std=0.5)
    pc = make_projection_case(2 * L - 1, F, H, d, dtype="bf16", basis="sinusoid", seed=24)
    X, W, _ = _dev(pc)
    pdesc = ear.make_proj_desc(2 * L - 1, F, H, d, dtype="bf16")
    desc = runner.desc_for(c)
    dev = runner.to_device(c)
    dev["rel_a"] = torch.empty((H, 2 * L - 1, d), dtype=torch.bfloat16, device="cuda")
    ear.relpos_project_fwd(pdesc, X, W, dev["rel_a"])
    o, lse = runner.forward(desc, dev)
    g = runner.backward(desc, dev, o, lse)
    dW = torch.empty((F, H * d), device="cuda")
    n = ear.relpos_project_workspace_size(pdesc)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    ear.relpos_project_bwd(pdesc, X, W, g["drel_a"], None, dW, ws, n)
    torch.cuda.synchronize()

    p = orc.Params(**c["params"])
    tab = {n_: t.astype(np.float64) for n_, t in c["tables"].items()}
    tab["r"] = prj.project(pc["X"], pc["W"], H, d)
    O_ref, lse_ref = orc.forward(p, c["q"], c["k"], c["v"], tab)
    tol = TOL["bf16"]
    assert np.max(np.abs(to_np(o) - O_ref)) <= tol["o"]
    _, _, _, gref = orc.backward(p, c["q"], c["k"], c["v"], tab, c["dout"])
    _, dW_ref = prj.project_backward(pc["X"], pc["W"], gref["r"])
    assert rel_l2(to_np(dW), dW_ref) <= tol["grad"], rel_l2(to_np(dW), dW_ref)


def test_deberta_projection_chained_with_attention():
    """Kr | Qr = P [W_r^k | W_r^q] in one call (two heads) feed the DeBERTa attention as rel_a,
    rel_b; its table gradients, written into the two halves of one [2, 2k, d] buffer, give dP
    (summed over both projections) and [dW_r^k | dW_r^q] in one backward call.  Checked against
    the oracle at L = 512, span 128, B = 1, H = 2."""
    import torch
    import exact_attention_relative_amd as ear
    from exact_attention_relative_amd import runner
    from exact_attention_relative_amd.inputs import make_case, make_projection_case
    from oracle import relpos_oracle as orc
    L, H, d, span = 512, 2, 64, 128
    c = make_case("deberta", 1, H, L, d, dtype="bf16", seed=31, rel_span=span)
    pc = make_projection_case(2 * span, d, 2, d, dtype="bf16", seed=32)
    X, W, _ = _dev(pc)
    pdesc = ear.make_proj_desc(2 * span, d, 2, d, dtype="bf16")
    rel = torch.empty((2, 2 * span, d), dtype=torch.bfloat16, device="cuda")
    ear.relpos_project_fwd(pdesc, X, W, rel)
    desc = runner.desc_for(c)
    dev = runner.to_device(c)
    dev["rel_a"], dev["rel_b"] = rel[0], rel[1]
    o, lse = runner.forward(desc, dev)
    drel = torch.empty((2, 2 * span, d), device="cuda")
    grads = runner.alloc_grads(desc, dev)
    grads["drel_a"], grads["drel_b"] = drel[0], drel[1]
    runner.backward(desc, dev, o, lse, grads=grads)
    dP = torch.empty((2 * span, d), device="cuda")
    dW = torch.empty((d, 2 * d), device="cuda")
    n = ear.relpos_project_workspace_size(pdesc)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    ear.relpos_project_bwd(pdesc, X, W, drel, dP, dW, ws, n)
    torch.cuda.synchronize()

    p = orc.Params(**c["params"])
    tab = {n_: t.astype(np.float64) for n_, t in c["tables"].items()}
    kq = prj.project(pc["X"], pc["W"], 2, d)
    tab["kr"], tab["qr"] = kq[0], kq[1]
    O_ref, _ = orc.forward(p, c["q"], c["k"], c["v"], tab)
    tol = TOL["bf16"]
    assert np.max(np.abs(to_np(o) - O_ref)) <= tol["o"]
    _, _, _, gref = orc.backward(p, c["q"], c["k"], c["v"], tab, c["dout"])
    dP_ref, dW_ref = prj.project_backward(pc["X"], pc["W"], np.stack([gref["kr"], gref["qr"]]))
    assert rel_l2(to_np(dP), dP_ref) <= tol["grad"], rel_l2(to_np(dP), dP_ref)
    assert rel_l2(to_np(dW), dW_ref) <= tol["grad"], rel_l2(to_np(dW), dW_ref)
