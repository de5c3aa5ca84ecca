"""fp64 cost matrices beyond the squared Euclidean one (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the product path never does.

Source: the page "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
(arXiv 2602.03067), §3.1 "Scope of cost structure": the streamed half-step
applies to any cost C_ij = alpha_i + beta_j - <Q_i, K_j> with per-point terms
alpha, beta and explicit features Q, K; the cosine cost is reached by
L2-normalising the points (1 - <x, y> = ||x - y||^2 / 2 for unit vectors);
§4.2 / App. H (OTDD) adds a label-to-label term W[l_i, l_j] to the feature
cost of each pair. Each function builds the dense matrix from its plain
definition; the Sinkhorn functions of ``oracle.sinkhorn`` take it as input.
"""

from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def cost_affine(alpha, beta, Q, K):
    """C_ij = alpha_i + beta_j - <Q_i, K_j> (§3.1 "Scope of cost structure")."""
    return _f64(alpha)[:, None] + _f64(beta)[None, :] - _f64(Q) @ _f64(K).T


def cost_cosine(X, Y):
    """Cosine cost C_ij = 1 - <x_i, y_j> / (||x_i|| ||y_j||) (§3.1). Points of
    zero norm have no direction; their rows / columns are set to 1 (the cost
    of orthogonal directions)."""
    X, Y = _f64(X), _f64(Y)
    nx = np.sqrt((X * X).sum(axis=1))
    ny = np.sqrt((Y * Y).sum(axis=1))
    Xh = np.divide(X, nx[:, None], out=np.zeros_like(X), where=nx[:, None] > 0)
    Yh = np.divide(Y, ny[:, None], out=np.zeros_like(Y), where=ny[:, None] > 0)
    return 1.0 - Xh @ Yh.T


def cost_labels(X, Y, lx, ly, W):
    """Label-augmented cost C_ij = ||x_i - y_j||^2 + W[l_i, l_j] (the OTDD cost of
    §4.2: feature distance plus a label-to-label term), written pair by pair
    with the direct difference."""
    X, Y, W = _f64(X), _f64(Y), _f64(W)
    lx = np.asarray(lx)
    ly = np.asarray(ly)
    D = X[:, None, :] - Y[None, :, :]
    return (D * D).sum(axis=2) + W[lx[:, None], ly[None, :]]
