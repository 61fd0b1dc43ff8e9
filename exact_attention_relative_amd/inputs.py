"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random tensors and prepares relation tables.  It holds none of the
attention arithmetic: it does not compute scores, softmax or gradients.  Both the fp64
oracle and the HIP library receive exactly the arrays it returns.

Recipe (the pages publish no shapes; the workloads below stand in for their
"8K-token sequences"):
  * numpy.random.default_rng(seed) (PCG64); every tensor drawn as float32 standard
    normals and multiplied by its standard deviation in float32;
  * draw order: Q, K, V, dO, then the relation tables of the mechanism;
  * bf16 workloads round every bf16 tensor to bf16 by round-to-nearest-even and keep
    the rounded values (stored in float32 arrays), so both sides see identical inputs;
  * T5 beta and T-XL u, v stay float32 in every mode;
  * T-XL r = R W_r with R the sinusoid [sin(delta w_m) | cos(delta w_m)],
    w_m = 10000^(-2m/512), m < 256, at every table offset delta, and
    W_r [512, H d] ~ N(0, 1/512); head h takes columns h d .. h d + d - 1;
  * DeBERTa Kr = P W_r^k and Qr = P W_r^q with P [2k, d] ~ N(0, table_std^2) and
    W_r^{k,q} [d, d] ~ N(0, 1/d) (row-vector convention);
  * ALiBi slopes m_h = 2^(-8 (h + 1) / H), the original geometric sequence (no draw;
    parity variants scale them by 1 + 4 table_std);
  * relation-table layout: by default Shaw's w and DeBERTa's Kr, Qr are shared by every head
    and T-XL has one r per head; rel_layout="per_head" draws one w / P per head (leading head
    axis; T-XL unchanged) and rel_layout="shared" gives T-XL one r for every head (W_r
    [512, d]; Shaw and DeBERTa unchanged).
  The projections are input preparation, done in float64 and rounded to the input
  dtype; the attention library takes r, Kr, Qr as given.
"""

from __future__ import annotations

import math

import numpy as np

# name -> workload description.  "window" is (window_left, window_right).
CONFIGS = {
    "t5_fp32_L128": dict(mech="t5", B=1, H=1, L=128, d=64, dtype="fp32", window=(-1, -1),
                         num_buckets=32, max_distance=128, bidirectional=True, seed=0,
                         passes=("fwd",)),
    "shaw_causal_L1024": dict(mech="shaw", B=2, H=8, L=1024, d=64, dtype="bf16", window=(-1, 0),
                              rel_span=128, seed=1, passes=("fwd", "bwd")),
    "deberta_L2048": dict(mech="deberta", B=2, H=12, L=2048, d=64, dtype="bf16", window=(-1, -1),
                          rel_span=256, seed=2, passes=("fwd", "bwd")),
    "txl_causal_L8192": dict(mech="txl", B=1, H=8, L=8192, d=64, dtype="bf16", window=(-1, 0),
                             seed=3, passes=("fwd", "bwd")),
    "long_t5_L8192": dict(mech="t5", B=4, H=8, L=8192, d=64, dtype="bf16", window=(-1, -1),
                          num_buckets=32, max_distance=1024, bidirectional=True, seed=5,
                          sub=0, passes=("fwd", "bwd")),
    "long_shaw_L8192": dict(mech="shaw", B=4, H=8, L=8192, d=64, dtype="bf16", window=(-1, -1),
                            rel_span=256, seed=5, sub=1, passes=("fwd", "bwd")),
    "long_deberta_L8192": dict(mech="deberta", B=4, H=8, L=8192, d=64, dtype="bf16",
                               window=(-1, -1), rel_span=512, seed=5, sub=2,
                               passes=("fwd", "bwd")),
    "long_txl_L8192": dict(mech="txl", B=4, H=8, L=8192, d=64, dtype="bf16", window=(-1, -1),
                           seed=5, sub=3, passes=("fwd", "bwd")),
}

LONG_WORKLOAD = ("long_t5_L8192", "long_shaw_L8192", "long_deberta_L8192", "long_txl_L8192")


def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    return (r.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _rng(seed: int, sub: int | None):
    if sub is None:
        return np.random.default_rng(seed)
    return np.random.default_rng([seed, sub])


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return round_bf16(x) if dtype == "bf16" else x


def sinusoid(offsets: np.ndarray, d_model: int = 512) -> np.ndarray:
    """[len(offsets), d_model] float64: sin(delta w_m) | cos(delta w_m)."""
    half = d_model // 2
    m = np.arange(half, dtype=np.float64)
    w = 10000.0 ** (-2.0 * m / d_model)
    ang = offsets.astype(np.float64)[:, None] * w[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)


def make_case(mech: str, B: int, H: int, L: int, d: int, *, dtype: str = "bf16",
              window=(-1, -1), seed: int = 0, sub: int | None = None, num_buckets: int = 32,
              max_distance: int = 128, bidirectional: bool | None = None, rel_span: int = 0,
              table_std: float | None = None, bias_std: float = 0.5, with_dout: bool = True,
              rel_layout: str | None = None, **_ignored) -> dict:
    """Draw one workload.  Returns dict(q, k, v, dout, tables, params) of numpy arrays."""
    rng = _rng(seed, sub)
    wl, wr = window
    causal = wr == 0
    if bidirectional is None:
        bidirectional = not causal
    shp = (B, H, L, d)
    q = _normal(rng, shp, 1.0, dtype)
    k = _normal(rng, shp, 1.0, dtype)
    v = _normal(rng, shp, 1.0, dtype)
    dout = _normal(rng, shp, 1.0, dtype) if with_dout else None
    tables = {}
    raw = {}
    tstd = 0.02 if table_std is None else table_std
    if mech == "t5":
        tables["beta"] = rng.standard_normal((H, num_buckets), dtype=np.float32) * np.float32(bias_std)
    elif mech == "shaw":
        lead = (H,) if rel_layout == "per_head" else ()
        tables["w"] = _normal(rng, lead + (2 * rel_span + 1, d), tstd, dtype)
    elif mech == "txl":
        nrel = L if causal else 2 * L - 1
        offsets = np.arange(nrel) if causal else np.arange(-(L - 1), L)
        hr = 1 if rel_layout == "shared" else H
        w_r = rng.standard_normal((512, hr * d), dtype=np.float32) * np.float32(1.0 / math.sqrt(512))
        r = (sinusoid(offsets) @ w_r.astype(np.float64)).astype(np.float32)
        r = r.reshape(nrel, hr, d).transpose(1, 0, 2)
        if rel_layout == "shared":
            r = r[0]
        tables["r"] = np.ascontiguousarray(round_bf16(r) if dtype == "bf16" else r)
        tables["u"] = rng.standard_normal((H, d), dtype=np.float32) * np.float32(tstd)
        tables["v"] = rng.standard_normal((H, d), dtype=np.float32) * np.float32(tstd)
        raw["w_r"] = w_r
    elif mech == "deberta":
        lead = (H,) if rel_layout == "per_head" else ()
        P = _normal(rng, lead + (2 * rel_span, d), tstd, dtype)
        wq = rng.standard_normal((d, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
        wk = rng.standard_normal((d, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
        kr = (P.astype(np.float64) @ wk.astype(np.float64)).astype(np.float32)
        qr = (P.astype(np.float64) @ wq.astype(np.float64)).astype(np.float32)
        tables["kr"] = round_bf16(kr) if dtype == "bf16" else kr
        tables["qr"] = round_bf16(qr) if dtype == "bf16" else qr
        raw.update(P=P, w_q=wq, w_k=wk)
    elif mech == "alibi":
        # the geometric per-head slopes 2^(-8 (h + 1) / H) of the original ALiBi recipe
        tables["slopes"] = np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)
        if table_std is not None:   # parity variants: larger, head-varied slopes
            tables["slopes"] = tables["slopes"] * np.float32(1.0 + 4.0 * table_std)
    else:
        raise ValueError(mech)
    params = dict(mech=mech, head_dim=d, window_left=wl, window_right=wr,
                  num_buckets=num_buckets, max_distance=max_distance,
                  bidirectional=bool(bidirectional), rel_span=rel_span)
    return dict(q=q, k=k, v=v, dout=dout, tables=tables, params=params, raw=raw,
                dtype=dtype, shape=shp)


def make_projection_case(N: int, F: int, H: int, d: int, *, dtype: str = "bf16",
                         basis: str = "normal", first_offset: int | None = None, seed: int = 0,
                         sub: int | None = None) -> dict:
    """Draw a relation-table projection workload: the basis X [N, F], the weight W [F, H d]
    (both rounded to bf16 when dtype is bf16) and an fp32 table gradient drel [H, N, d].

    basis "sinusoid": the sin | cos features of N consecutive offsets from `first_offset`
    (default -(N-1)//2, the full span; 0 for the causal table), T-XL's R with values in
    [-1, 1] and F even; "normal": N(0, 0.02^2) rows (a learned DeBERTa P)."""
    rng = _rng(seed, sub)
    if basis == "sinusoid":
        start = -((N - 1) // 2) if first_offset is None else first_offset
        offsets = np.arange(N, dtype=np.int64) + start
        X = sinusoid(offsets, F).astype(np.float32)
        X = round_bf16(X) if dtype == "bf16" else X
    else:
        X = _normal(rng, (N, F), 0.02, dtype)
    W = _normal(rng, (F, H * d), 1.0 / math.sqrt(F), dtype)
    drel = rng.standard_normal((H, N, d), dtype=np.float32) * np.float32(1e-3)
    return dict(X=np.ascontiguousarray(X), W=W, drel=drel, shape=(N, F, H, d), dtype=dtype)


def make_config(name: str, **overrides) -> dict:
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    case = make_case(**cfg)
    case["config"] = cfg
    return case
