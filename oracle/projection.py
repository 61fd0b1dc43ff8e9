"""fp64 CPU oracle of the relation-table projections (test infrastructure only).

The relation tables of T-XL and DeBERTa are projections of a position basis: T-XL
r = R W_r (R the sinusoid features of every offset) and DeBERTa Kr = P W_r^k, Qr = P W_r^q.
The explainer's section on reusing query-key relation products treats such decomposable
"bias vector x position embedding" terms; the projections themselves are the original
mechanisms' definitions, written here as plain matrix products:

    rel[h][n][c] = sum_f X[n][f] W[f][h d + c]            (H heads of width d; H = 1 for DeBERTa)
    dW[f][h d + c] = sum_n X[n][f] drel[h][n][c]
    dX[n][f]       = sum_{h, c} drel[h][n][c] W[f][h d + c]

Only the tests, the smoke check and the bench's CPU leg may use this module.
Pins: tests/test_oracle_pins.py (scalar loops at small sizes, central differences).
"""

from __future__ import annotations

import numpy as np


def project(X, W, H: int, d: int) -> np.ndarray:
    """rel [H, N, d] from X [N, F] and W [F, H d], in float64."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    N = X.shape[0]
    return (X @ W).reshape(N, H, d).transpose(1, 0, 2)


def project_backward(X, W, drel):
    """(dX [N, F], dW [F, H d]) from drel [H, N, d], in float64."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    drel = np.asarray(drel, dtype=np.float64)
    H, N, d = drel.shape
    dY = drel.transpose(1, 0, 2).reshape(N, H * d)
    return dY @ W.T, X.T @ dY
