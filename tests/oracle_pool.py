"""The fp64 oracle's long-sequence outputs over a pool of worker processes (test helper).

Each task is a contiguous range of query rows of one (batch, head) slice: a worker runs the
oracle's backward_chunk over it `chunk` rows at a time and merges the parts in ascending order
(sum_chunks); the parent merges the tasks of a slice in ascending order and finishes them
(finish_chunks).  The result is the oracle's backward up to the order of fp64 sums.  Workers are
spawned (they inherit no GPU state), use one BLAS thread each, and number at most 16."""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

_W: dict = {}


def _init(arrays, params, tables):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:   # pragma: no cover
        pass
    _W.update(arrays=arrays, params=params, tables=tables)


def _task(args):
    b, h, lo, hi, chunk = args
    from oracle import relpos_oracle as orc
    a = _W["arrays"]
    p = orc.Params(**_W["params"])
    parts = [orc.backward_chunk(p, a["q"], a["k"], a["v"], _W["tables"], a["dout"], b, h,
                                np.arange(r0, min(hi, r0 + chunk)))
             for r0 in range(lo, hi, chunk)]
    return b, h, lo, orc.sum_chunks(parts)


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_long(case: dict, slices, chunk: int = 256, nproc: int | None = None) -> dict:
    """O, LSE, dq, dk, dv for every (b, h) in `slices` and the table gradients summed over those
    slices (per-head tables at their head).  Returns {"o": {(b,h): [L, d]}, ..., "g": {...}}."""
    from oracle import relpos_oracle as orc
    p = orc.Params(**case["params"])
    tables = {n: t.astype(np.float64) for n, t in case["tables"].items()}
    arrays = {n: case[n] for n in ("q", "k", "v", "dout")}
    L = case["q"].shape[2]
    nproc = nproc or workers()
    per = -(-L // nproc)
    per = -(-per // chunk) * chunk
    tasks = [(b, h, lo, min(L, lo + per), chunk) for (b, h) in slices for lo in range(0, L, per)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(nproc, initializer=_init, initargs=(arrays, case["params"], tables)) as pool:
        done = pool.map(_task, tasks, chunksize=1)
    out = {"o": {}, "lse": {}, "dq": {}, "dk": {}, "dv": {},
           "g": {n: np.zeros(np.shape(t)) for n, t in tables.items()}}
    for (b, h) in slices:
        mine = sorted((r for r in done if r[0] == b and r[1] == h), key=lambda r: r[2])
        merged = orc.sum_chunks([r[3] for r in mine])
        dq, dk, dv, g = orc.finish_chunks(p, case["k"], tables, b, h, merged)
        o = np.zeros((L, case["q"].shape[3]))
        lse = np.zeros(L)
        o[merged["rows"]] = merged["o"]
        lse[merged["rows"]] = merged["lse"]
        out["o"][(b, h)], out["lse"][(b, h)] = o, lse
        out["dq"][(b, h)], out["dk"][(b, h)], out["dv"][(b, h)] = dq, dk, dv
        orc.add_table_grads(out["g"], g, tables, h)
    return out
