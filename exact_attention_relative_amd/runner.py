"""Torch plumbing around the C ABI: device buffers for a workload, output allocation and the
pass sequence.  No arithmetic of the method happens here."""

from __future__ import annotations

import numpy as np
import torch

from . import (make_desc, relpos_attn_bwd, relpos_attn_fwd, relpos_attn_workspace_size)

# which table goes in which C-ABI slot, per mechanism
SLOTS = {
    "t5": {"bias_a": "beta"},
    "shaw": {"rel_a": "w"},
    "txl": {"rel_a": "r", "bias_a": "u", "bias_b": "v"},
    "deberta": {"rel_a": "kr", "rel_b": "qr"},
    "alibi": {"bias_a": "slopes"},
}
# gradient slot of each table
GRAD_SLOTS = {"rel_a": "drel_a", "rel_b": "drel_b", "bias_a": "dbias_a", "bias_b": "dbias_b"}


def tensor_from_f32(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """float32 numpy values (bf16-representable when dtype is bf16) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)   # exact: the values are already bf16
    return t.to(device)


# relation tables (head axis optional: a table with one more axis than these is per head)
REL_TABLES = {"shaw": ("w",), "txl": ("r",), "deberta": ("kr", "qr")}
REL_NDIM = {"w": 2, "r": 2, "kr": 2, "qr": 2}


def rel_head_stride(case: dict) -> int:
    """0 when the case's relation tables are shared by every head, else the elements between
    consecutive heads' tables (dense [H, rows, d])."""
    names = REL_TABLES.get(case["params"]["mech"], ())
    for n in names:
        t = case["tables"][n]
        if t.ndim == REL_NDIM[n] + 1:
            return int(t.shape[1] * t.shape[2])
    return 0


def desc_for(case: dict, **overrides):
    p = case["params"]
    B, H, L, d = case["shape"]
    kw = dict(dtype=case["dtype"], window=(p["window_left"], p["window_right"]),
              rel_span=p["rel_span"], num_buckets=p["num_buckets"],
              max_distance=p["max_distance"], bidirectional=p["bidirectional"],
              scale=p.get("scale", 0.0) or 0.0, rel_head_stride=rel_head_stride(case))
    kw.update(overrides)
    return make_desc(p["mech"], B, H, L, d, **kw)


def to_device(case: dict, device="cuda") -> dict:
    dt = case["dtype"]
    mech = case["params"]["mech"]
    dev = {n: tensor_from_f32(case[n], dt, device) for n in ("q", "k", "v")}
    if case.get("dout") is not None:
        dev["dout"] = tensor_from_f32(case["dout"], dt, device)
    for slot, name in SLOTS[mech].items():
        fp32_table = name in ("beta", "u", "v", "slopes")
        dev[slot] = tensor_from_f32(case["tables"][name], "fp32" if fp32_table else dt, device)
    return dev


def slots(dev):
    return tuple(dev.get(s) for s in ("rel_a", "rel_b", "bias_a", "bias_b"))


def workspace(desc, pass_, device="cuda"):
    n = relpos_attn_workspace_size(desc, pass_)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def forward(desc, dev, ws=None):
    q = dev["q"]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    if ws is None:
        ws, n = workspace(desc, 0, q.device)
    else:
        n = ws.numel()
    relpos_attn_fwd(desc, q, dev["k"], dev["v"], *slots(dev), o, lse, ws, n)
    return o, lse


def alloc_grads(desc, dev):
    q = dev["q"]
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(q), "dv": torch.empty_like(q)}
    for slot, gname in GRAD_SLOTS.items():
        if dev.get(slot) is not None:
            g[gname] = torch.empty(dev[slot].shape, dtype=torch.float32, device=q.device)
    return g


def backward(desc, dev, o, lse, ws=None, grads=None):
    if grads is None:
        grads = alloc_grads(desc, dev)
    if ws is None:
        ws, n = workspace(desc, 1, dev["q"].device)
    else:
        n = ws.numel()
    relpos_attn_bwd(desc, dev["q"], dev["k"], dev["v"], o, lse, dev["dout"], *slots(dev),
                    grads["dq"], grads["dk"], grads["dv"], grads.get("drel_a"), grads.get("drel_b"),
                    grads.get("dbias_a"), grads.get("dbias_b"), ws, n)
    return grads


def named_table_grads(mech: str, grads: dict) -> dict:
    """Map slot gradients back to table names (e.g. drel_a -> 'w' for Shaw)."""
    out = {}
    for slot, name in SLOTS[mech].items():
        out[name] = grads[GRAD_SLOTS[slot]]
    return out
