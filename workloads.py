"""Seeded synthetic workloads for the streamed Sinkhorn solver.

This module only draws random inputs: point clouds, weights and the value
matrices that the transport-application step multiplies. It contains none of
the solver's arithmetic and is shared by the tests, ``bench.py`` and the
smoke check, so that the HIP path and the fp64 oracle see identical arrays.

Shapes and distributions follow the five benchmark configurations this
project is measured on. They stand in for the page's own synthetic point
clouds ("FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", App. H.2:
uniform points in [0,1]^d, n in [5k, 50k], d in [4, 1024]) and, for the
70000 x 512 mixture, for the MNIST / Fashion-MNIST embedding shapes of §4.2,
whose data is not available here.

Recipe (every array drawn in float64 with ``numpy.random.default_rng``, then
rounded to float32; bf16 workloads round the float32 values once more to
bfloat16 with round-to-nearest-even and keep them as float32 holding exactly
representable values):

  seed(array) = 1000 * config + 10 * variant + index,
  index: x=0, y=1, a=2, b=3, V=4, U=5, x-mixture means=6, y-mixture means=7,
         x labels=8, y labels=9, HVP direction A=10.

The Hessian-vector-product workload follows the page's own HVP benchmark
(App. H.2: points uniform in [0,1]^d, uniform marginals, eps = 0.1, 100
Sinkhorn iterations, then conjugate gradients with K = 50, tau = 1e-5), at
its largest size n = m = 50000, d = 64, with a direction A ~ N(0, 1).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_IDX = dict(x=0, y=1, a=2, b=3, V=4, U=5, mx=6, my=7, lx=8, ly=9, A=10)


@dataclass(frozen=True)
class Workload:
    name: str
    config: int
    variant: int
    n: int
    m: int
    d: int
    dtype: str              # "f32" or "bf16": storage type of X and Y
    eps: float
    iters: int
    xdist: str
    ydist: str
    weights: str            # "uniform" | "dirichlet" | "lognormal"
    v_cols: int = 0         # P V with V (m x v_cols) ~ N(0,1); 0 = none
    u_cols: int = 0         # P^T U with U (n x u_cols) ~ N(0,1); 0 = none
    grad: bool = False      # P Y -> gradient in X
    extra: dict = field(default_factory=dict)


def _c3(variant, d, dtype):
    return Workload(f"c3_d{d}_{dtype}", 3, variant, 20000, 20000, d, dtype, 0.1, 100,
                    "gauss", "gauss_shift", "dirichlet")


WORKLOADS = {
    # n=m=1024, d=16, fp32, eps=0.1, 50 iterations; f, g and marginal error.
    "c1": Workload("c1", 1, 0, 1024, 1024, 16, "f32", 0.1, 50,
                   "gauss", "gauss_shift", "uniform"),
    # n=m=20000, d=64, fp32, eps=0.1, 100 iterations; then P Y -> grad_x.
    "c2": Workload("c2", 2, 0, 20000, 20000, 64, "f32", 0.1, 100,
                   "gauss", "gauss_shift", "uniform", grad=True),
    # n=m=20000, d in {16,128,512,1024} x {fp32, bf16}; Dirichlet(1) weights.
    "c3_d16_f32": _c3(0, 16, "f32"),
    "c3_d128_f32": _c3(1, 128, "f32"),
    "c3_d512_f32": _c3(2, 512, "f32"),
    "c3_d1024_f32": _c3(3, 1024, "f32"),
    "c3_d16_bf16": _c3(4, 16, "bf16"),
    "c3_d128_bf16": _c3(5, 128, "bf16"),
    "c3_d512_bf16": _c3(6, 512, "bf16"),
    "c3_d1024_bf16": _c3(7, 1024, "bf16"),
    # n=m=70000, d=512, bf16, 10-component mixtures, 200 iterations; P V (m x 64).
    "c4": Workload("c4", 4, 0, 70000, 70000, 512, "bf16", 0.1, 200,
                   "mixture", "mixture", "uniform", v_cols=64),
    # n=200000, m=10000, d=1024, fp32, eps=0.01, 300 iterations; P V and P^T U.
    "c5": Workload("c5", 5, 0, 200000, 10000, 1024, "f32", 0.01, 300,
                   "gauss", "uniform_box", "lognormal", v_cols=128, u_cols=128),
    # Hessian-vector product: n=m=50000, d=64, uniform [0,1]^d points, eps=0.1,
    # 100 iterations, then CG with K=50, tau=1e-5 (direction A ~ N(0,1)).
    "hvp_n50k_d64": Workload("hvp_n50k_d64", 6, 0, 50000, 50000, 64, "f32", 0.1, 100,
                             "unit_box", "unit_box", "uniform", extra={"hvp_A": True}),
}


def _rng(w: Workload, key: str) -> np.random.Generator:
    return np.random.default_rng(1000 * w.config + 10 * w.variant + _IDX[key])


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def _points(w: Workload, rows: int, dist: str, key: str, mkey: str, lkey: str) -> np.ndarray:
    d = w.d
    s = 1.0 / math.sqrt(d) if d > 0 else 1.0
    rng = _rng(w, key)
    if dist == "gauss":                    # N(0, I_d) / sqrt(d)
        P = rng.standard_normal((rows, d)) * s
    elif dist == "gauss_shift":            # (N(0, I_d) + 1) / sqrt(d): unit mean shift
        P = (rng.standard_normal((rows, d)) + 1.0) * s
    elif dist == "unit_box":               # Uniform[0, 1]^d (page's synthetic benchmark points)
        P = rng.uniform(0.0, 1.0, (rows, d))
    elif dist == "uniform_box":            # Uniform[-1, 1]^d / sqrt(d)
        P = rng.uniform(-1.0, 1.0, (rows, d)) * s
    elif dist == "mixture":                # 10 components, means ~ N(0, 4 I)/sqrt(d), std 0.5/sqrt(d)
        means = _rng(w, mkey).standard_normal((10, d)) * (2.0 * s)
        labels = _rng(w, lkey).integers(0, 10, rows)
        P = means[labels] + rng.standard_normal((rows, d)) * (0.5 * s)
    else:
        raise ValueError(dist)
    return P


def _weights(w: Workload, rows: int, key: str) -> np.ndarray:
    if w.weights == "uniform":
        return np.full(rows, 1.0 / rows)
    rng = _rng(w, key)
    if w.weights == "dirichlet":           # Dirichlet(1) = normalised i.i.d. Exp(1)
        v = rng.exponential(1.0, rows)
    elif w.weights == "lognormal":         # log-normal(0, 1), normalised
        v = rng.lognormal(0.0, 1.0, rows)
    else:
        raise ValueError(w.weights)
    return v / v.sum()


def make(name: str, n: int | None = None, m: int | None = None, d: int | None = None,
         v_cols: int | None = None, u_cols: int | None = None) -> dict:
    """Draw the arrays of workload ``name`` (optionally resized, same distributions).

    Returns a dict with float32 numpy arrays X (n x d), Y (m x d), a (n), b (m),
    V (m x v_cols) and U (n x u_cols) when requested, plus the Workload record
    under "w" (with n, m, d replaced by the sizes actually drawn).
    """
    base = WORKLOADS[name]
    n = base.n if n is None else int(n)
    m = base.m if m is None else int(m)
    d = base.d if d is None else int(d)
    v_cols = base.v_cols if v_cols is None else int(v_cols)
    u_cols = base.u_cols if u_cols is None else int(u_cols)
    w = Workload(base.name, base.config, base.variant, n, m, d, base.dtype, base.eps,
                 base.iters, base.xdist, base.ydist, base.weights, v_cols, u_cols,
                 base.grad, dict(base.extra))
    X = _points(w, n, w.xdist, "x", "mx", "lx").astype(np.float32)
    Y = _points(w, m, w.ydist, "y", "my", "ly").astype(np.float32)
    if w.dtype == "bf16":
        X = bf16_round(X)
        Y = bf16_round(Y)
    out = dict(w=w, X=X, Y=Y,
               a=_weights(w, n, "a").astype(np.float32),
               b=_weights(w, m, "b").astype(np.float32))
    if v_cols:
        V = _rng(w, "V").standard_normal((m, v_cols)).astype(np.float32)
        out["V"] = bf16_round(V) if w.dtype == "bf16" else V
    if u_cols:
        U = _rng(w, "U").standard_normal((n, u_cols)).astype(np.float32)
        out["U"] = bf16_round(U) if w.dtype == "bf16" else U
    if w.extra.get("hvp_A"):
        out["A"] = _rng(w, "A").standard_normal((n, d)).astype(np.float32)
    return out


def hvp_parity_inputs(n: int, m: int, d: int, seed: int) -> dict:
    """Inputs of the Hessian-vector-product parity protocol of the page (App. H.2.3
    "HVP Parity": X, Y ~ N(0, I_d), a, b random simplex weights), plus the
    direction A ~ N(0, I) (n x d). float32 arrays X, Y, A, a, b."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((m, d))
    a = rng.exponential(1.0, n)
    b = rng.exponential(1.0, m)
    A = rng.standard_normal((n, d))
    f32 = lambda v: np.ascontiguousarray(v, dtype=np.float32)
    return dict(X=f32(X), Y=f32(Y), A=f32(A), a=f32(a / a.sum()), b=f32(b / b.sum()))


def potential_offsets(n: int, m: int, seed: int, scale: float = 0.1) -> tuple[np.ndarray, np.ndarray]:
    """Seeded offsets u (n), v (m) ~ scale * N(0, 1), float32: test potentials are
    formed as f = ||x||^2 + u, g = ||y||^2 + v, so that both sides of a
    teacher-forced check receive the same realistic-scale inputs."""
    rng = np.random.default_rng(seed)
    return ((rng.standard_normal(n) * scale).astype(np.float32),
            (rng.standard_normal(m) * scale).astype(np.float32))


def affine_inputs(n: int, m: int, d: int, seed: int) -> dict:
    """Seeded inputs of a general affine cost alpha_i + beta_j - <Q_i, K_j> (§3.1
    "Scope of cost structure"): features Q, K ~ N(0, I_d) / sqrt(d), offsets
    alpha, beta ~ Uniform[0, 1], Dirichlet(1) weights. float32 arrays."""
    rng = np.random.default_rng(seed)
    s = 1.0 / math.sqrt(d)
    f32 = lambda v: np.ascontiguousarray(v, dtype=np.float32)
    a = rng.exponential(1.0, n)
    b = rng.exponential(1.0, m)
    return dict(Q=f32(rng.standard_normal((n, d)) * s), K=f32(rng.standard_normal((m, d)) * s),
                alpha=f32(rng.uniform(0.0, 1.0, n)), beta=f32(rng.uniform(0.0, 1.0, m)),
                a=f32(a / a.sum()), b=f32(b / b.sum()))


def label_inputs(n: int, m: int, n_labels: int, seed: int) -> dict:
    """Seeded class labels (uniform over n_labels classes) and a symmetric
    label-to-label cost W with zero diagonal and entries ~ Uniform[0.5, 2]
    off it, standing in for the OTDD label distances of §4.2 (whose embedding
    data is not available). int32 labels, float32 W."""
    rng = np.random.default_rng(seed)
    W = rng.uniform(0.5, 2.0, (n_labels, n_labels))
    W = 0.5 * (W + W.T)
    np.fill_diagonal(W, 0.0)
    return dict(lx=rng.integers(0, n_labels, n).astype(np.int32),
                ly=rng.integers(0, n_labels, m).astype(np.int32),
                W=np.ascontiguousarray(W, dtype=np.float32))
