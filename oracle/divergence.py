"""fp64 reference of eps-scaling and the debiased Sinkhorn divergence
(TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the product path never does.

Source: the page "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
(arXiv 2602.03067). The page names both only as options its benchmarks turn
off (App. H.2: "no epsilon-scaling", "no debiasing") and as the quantity
users evaluate (§1: the Sinkhorn divergence at MNIST scale); it gives no
formula. The readings implemented here are the plainest ones consistent
with the rest of the page:

* eps-scaling: iteration k of the alternating schedule (§3.1 eq. 2-3) runs
  at eps_k = max(eps, eps_start * decay^k), a geometric decrease from
  eps_start to the target eps, after which every iteration runs at eps;
* the entropic OT value of a pair of measures is the dual value
  <a, f> + <b, g> of the potentials after the iterations (§4.1: the forward
  pass returns potentials and cost);
* the debiased Sinkhorn divergence is
  S_eps(mu, nu) = OT_eps(mu, nu) - OT_eps(mu, mu) / 2 - OT_eps(nu, nu) / 2,
  each term solved with the same schedule and iteration count.
"""

from __future__ import annotations

import numpy as np

from .sinkhorn import cost_matrix, dual_value, sinkhorn, update_f, update_g


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def eps_schedule(eps, iters, eps_start=0.0, decay=0.5):
    """The eps of each iteration: max(eps, eps_start * decay^k) (eps_start <= eps: all eps)."""
    out = []
    for k in range(int(iters)):
        e = eps_start * decay ** k if eps_start > eps else eps
        out.append(max(eps, e))
    return out


def sinkhorn_eps_scaling(C, a, b, eps, iters, eps_start, decay, f0=None, g0=None,
                         schedule="alternating"):
    """Sinkhorn where iteration k runs both half-steps at eps_k of ``eps_schedule``
    (the potentials carry over from one eps to the next). schedule
    "alternating": f from g, then g from the new f (§3.1 eq. 2-3);
    "symmetric": both from the previous iterate, averaged (eq. 4-5)."""
    C = _f64(C)
    n, m = C.shape
    f = np.zeros(n) if f0 is None else _f64(f0).copy()
    g = np.zeros(m) if g0 is None else _f64(g0).copy()
    for e in eps_schedule(eps, iters, eps_start, decay):
        if schedule == "symmetric":
            ft = update_f(C, g, b, e)
            gt = update_g(C, f, a, e)
            f, g = 0.5 * (f + ft), 0.5 * (g + gt)
        else:
            f = update_f(C, g, b, e)
            g = update_g(C, f, a, e)
    return f, g


def _solve(C, a, b, eps, iters, eps_start, decay, schedule):
    if eps_start > eps or schedule == "symmetric":
        return sinkhorn_eps_scaling(C, a, b, eps, iters, eps_start, decay, schedule=schedule)
    return sinkhorn(C, a, b, eps, iters)


def sinkhorn_divergence(X, Y, a, b, eps, iters, eps_start=0.0, decay=0.5, schedule="alternating"):
    """S_eps(mu, nu) = OT(mu, nu) - OT(mu, mu)/2 - OT(nu, nu)/2 with each OT the dual
    value of its own solve (same schedule, eps, iterations and eps-scaling).

    Returns (S, OT(mu, nu), OT(mu, mu), OT(nu, nu), f, g, f_xx, g_yy) where
    (f, g) solve (mu, nu), f_xx is the f-side potential of (mu, mu) and g_yy
    the g-side potential of (nu, nu)."""
    X, Y, a, b = _f64(X), _f64(Y), _f64(a), _f64(b)
    f, g = _solve(cost_matrix(X, Y), a, b, eps, iters, eps_start, decay, schedule)
    fxx, gxx = _solve(cost_matrix(X, X), a, a, eps, iters, eps_start, decay, schedule)
    fyy, gyy = _solve(cost_matrix(Y, Y), b, b, eps, iters, eps_start, decay, schedule)
    ot_xy = dual_value(a, b, f, g)
    ot_xx = dual_value(a, a, fxx, gxx)
    ot_yy = dual_value(b, b, fyy, gyy)
    return ot_xy - 0.5 * ot_xx - 0.5 * ot_yy, ot_xy, ot_xx, ot_yy, f, g, fxx, gyy
