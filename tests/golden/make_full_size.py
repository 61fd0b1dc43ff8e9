"""Writes tests/golden/full_<workload>.npz: fp64 oracle values at the full workload sizes.

Only oracle/ and the seeded input generator are used.  Stored (as float32):
  o, lse, dq, dk, dv  at sampled (batch, head) slices and sampled rows,
  every table gradient (T-XL r at sampled offset rows, u and v in full).

    python tests/golden/make_full_size.py [workload ...]   (about 30 min on 8 cores)
"""

from __future__ import annotations

import multiprocessing as mp
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

WORKLOADS = ["shaw_causal_L1024", "deberta_L2048", "txl_causal_L8192", "long_t5_L8192",
             "long_shaw_L8192", "long_deberta_L8192", "long_txl_L8192"]


def sample_plan(B, H, L):
    """(batch, head) slices and rows checked one by one at full size."""
    bh = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 3), ((B - 1) // 2, (2 * H) // 3)})
    rows = np.unique(np.concatenate([np.linspace(0, L - 1, 48).astype(np.int64),
                                     np.array([0, 1, 2, 63, 64, 127, 128, L // 2, L - 2, L - 1])]))
    return bh, rows


def txl_sample_rows(nrel):
    return np.unique(np.linspace(0, nrel - 1, 192).astype(np.int64))


_CASE = None


def _init(name):
    global _CASE
    from exact_attention_relative_amd.inputs import make_config
    _CASE = make_config(name)


def _work(args):
    b, h, want = args
    from oracle import relpos_oracle as orc
    c = _CASE
    p = orc.Params(**c["params"])
    tab = {n: t.astype(np.float64) for n, t in c["tables"].items()}
    dq, dk, dv, g = orc.backward_head(p, c["q"], c["k"], c["v"], tab, c["dout"], b, h)
    out = {"g": g, "b": b, "h": h}
    if want is not None:
        O, lse = orc.forward_rows(p, c["q"], c["k"], c["v"], tab, b, h, want)
        out.update(o=O, lse=lse, dq=dq[want], dk=dk[want], dv=dv[want])
    return out


def make(name, procs=4):
    from exact_attention_relative_amd.inputs import CONFIGS, make_config
    from oracle import relpos_oracle as orc
    cfg = CONFIGS[name]
    B, H, L, d = cfg["B"], cfg["H"], cfg["L"], cfg["d"]
    bh, rows = sample_plan(B, H, L)
    jobs = [(b, h, rows if (b, h) in bh else None) for b in range(B) for h in range(H)]
    case = make_config(name)
    p = orc.Params(**case["params"])
    shapes = orc.table_shapes(p, H, L, d)
    grads = {n: np.zeros(s) for n, s in shapes.items()}
    samples = {}
    os.environ.setdefault("OMP_NUM_THREADS", "2")
    with mp.get_context("fork").Pool(procs, initializer=_init, initargs=(name,)) as pool:
        for res in pool.imap_unordered(_work, jobs):
            for n, v in res["g"].items():
                if n in ("beta", "r", "u", "v"):
                    grads[n][res["h"]] += v
                else:
                    grads[n] += v
            if "o" in res:
                samples[(res["b"], res["h"])] = res
            print(f"{name}: done b={res['b']} h={res['h']}", flush=True)
    out = {"bh": np.array(bh, dtype=np.int64), "rows": rows}
    for key in ("o", "lse", "dq", "dk", "dv"):
        out[key] = np.stack([samples[t][key] for t in bh]).astype(np.float32)
    for n, g in grads.items():
        if n == "r":
            sr = txl_sample_rows(g.shape[1])
            out["table_r_rows"] = sr
            out["table_r"] = g[:, sr].astype(np.float32)
        else:
            out["table_" + n] = g.astype(np.float32)
    np.savez_compressed(os.path.join(HERE, f"full_{name}.npz"), **out)


if __name__ == "__main__":
    names = sys.argv[1:] or WORKLOADS
    for n in names:
        make(n)
