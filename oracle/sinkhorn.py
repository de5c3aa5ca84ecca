"""fp64 reference definitions of the streamed Sinkhorn hot path (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the product path never does.

Source of every definition: the page "FlashSinkhorn: IO-Aware Entropic
Optimal Transport on GPU" (arXiv 2602.03067). Its display equations did not
survive on the page, so each function states the reading it implements:

* Measures: mu = sum_i a_i delta_{x_i}, nu = sum_j b_j delta_{y_j} with
  points X (n x d), Y (m x d) and positive weights a, b (used as given, not
  renormalised) -- §2.2 and App. H.2 (synthetic benchmarks).
* Cost: squared Euclidean C_ij = ||x_i - y_j||^2 -- §3.1 "Scope of cost
  structure" and App. H.2. Formed here by the direct difference.
* Potentials f (n), g (m) and the coupling
  P_ij = a_i b_j exp((f_i + g_j - C_ij) / eps). The a_i and b_j factors are
  fixed by App. E.1, whose induced marginal r = a * exp((f_hat - f_hat+)/eps)
  only holds with them; App. D.1 (delta = eps log b, gamma = eps log a) puts
  the log-weights inside the log-sum-exp the same way.
* Stabilised log-domain half-steps (§3.1, Prop. 1 / App. D.1):
    f_i <- -eps * LSE_j((g_j - C_ij)/eps + log b_j)
    g_j <- -eps * LSE_i((f_i - C_ij)/eps + log a_i)
* Alternating schedule (§3.1, eq. 2-3, the "OTT-style" updates of §4.1):
  each iteration updates f from the current g, then g from the new f.
  Iterations start from f = g = 0.
* Transport application (§3.2, Prop. 3, App. E.1): P V and P^T U of the
  coupling induced by ANY (f, g); its marginals r = P 1, c = P^T 1.
* Gradient (§2.2, §3.2, App. G.1 "Gradient", induced marginals):
  grad_X = sum_j P_ij * d/dx_i ||x_i - y_j||^2 = 2 (r * X - P Y).

No tiling, no online max/sum merge, no norm expansion: each function is the
plain definition, so that a reader can check it against the page by eye.
"""

from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sqnorms(P):
    """Row squared norms ||p_i||^2 (App. D.1: alpha_i = ||x_i||^2, beta_j = ||y_j||^2)."""
    P = _f64(P)
    return np.sum(P * P, axis=1)


def cost_matrix(X, Y, block_elems=1 << 24):
    """Squared-Euclidean cost C_ij = sum_k (x_ik - y_jk)^2 by the direct difference.

    §3.1 "Scope of cost structure" and App. H.2 fix the cost as ||x - y||^2.
    The sum runs over the coordinates of the difference vector; the
    ||x||^2 + ||y||^2 - 2 x.y expansion is deliberately not used here.
    """
    X = _f64(X)
    Y = _f64(Y)
    n, d = X.shape
    m, d2 = Y.shape
    assert d == d2, "X and Y must have the same dimension"
    C = np.empty((n, m), dtype=np.float64)
    if n == 0 or m == 0:
        return C
    rows = max(1, block_elems // max(1, m * max(d, 1)))
    for i0 in range(0, n, rows):
        diff = X[i0:i0 + rows, None, :] - Y[None, :, :]
        C[i0:i0 + rows] = np.einsum("ijk,ijk->ij", diff, diff)
    return C


def logsumexp(Z, axis):
    """LSE(z) = max z + log sum exp(z - max z) along ``axis`` (§2.3, App. D.3's target value)."""
    Z = _f64(Z)
    mx = np.max(Z, axis=axis, keepdims=True)
    s = np.sum(np.exp(Z - mx), axis=axis, keepdims=True)
    return np.squeeze(mx + np.log(s), axis=axis)


def update_f(C, g, b, eps):
    """f-half-step: f_i = -eps * LSE_j((g_j - C_ij)/eps + log b_j).

    §3.1 (stabilised alternating update, eq. 2) and Prop. 1 / App. D.1, which
    show the same value equals -eps * LSE_row of the biased dot-product score.
    """
    C = _f64(C)
    Z = (_f64(g)[None, :] - C) / eps + np.log(_f64(b))[None, :]
    return -eps * logsumexp(Z, axis=1)


def update_g(C, f, a, eps):
    """g-half-step: g_j = -eps * LSE_i((f_i - C_ij)/eps + log a_i).

    §3.1 (eq. 3) and App. D.1 ("the g-hat update ... can be proved similarly").
    """
    C = _f64(C)
    Z = (_f64(f)[:, None] - C) / eps + np.log(_f64(a))[:, None]
    return -eps * logsumexp(Z, axis=0)


def sinkhorn(C, a, b, eps, iters, f0=None, g0=None, record=False):
    """Alternating log-domain Sinkhorn for a fixed number of iterations.

    §3.1 (alternating schedule eq. 2-3) and §4.1 / App. H.2 (fixed iteration
    count, no early stopping, no eps-scaling). One iteration = one f
    half-step from the current g followed by one g half-step from the new f.
    Starts from f = g = 0 unless f0/g0 are given. With ``record`` the
    potentials after every iteration are returned as lists as well.
    """
    C = _f64(C)
    n, m = C.shape
    f = np.zeros(n) if f0 is None else _f64(f0).copy()
    g = np.zeros(m) if g0 is None else _f64(g0).copy()
    fs, gs = [], []
    for _ in range(int(iters)):
        f = update_f(C, g, b, eps)
        g = update_g(C, f, a, eps)
        if record:
            fs.append(f.copy())
            gs.append(g.copy())
    if record:
        return f, g, fs, gs
    return f, g


def sinkhorn_symmetric(C, a, b, eps, iters, f0=None, g0=None, record=False):
    """Symmetric (averaged) log-domain Sinkhorn for a fixed number of iterations.

    §3.1 (the symmetric updates eq. 4-5, fused "in the same single-kernel
    streaming form") and §4.1 / App. H.2 (the GeomLoss-style schedule, "flash(sym)").
    The equations did not survive on the page; the reading implemented here is
    the averaged update in which both half-steps read the previous iterate:

        f_new = (f + T_f(g)) / 2,   g_new = (g + T_g(f)) / 2,

    with T_f, T_g the half-steps of ``update_f`` / ``update_g``. Its fixed points
    are those of the alternating schedule. Starts from f = g = 0 unless given.
    """
    C = _f64(C)
    n, m = C.shape
    f = np.zeros(n) if f0 is None else _f64(f0).copy()
    g = np.zeros(m) if g0 is None else _f64(g0).copy()
    fs, gs = [], []
    for _ in range(int(iters)):
        ft = update_f(C, g, b, eps)
        gt = update_g(C, f, a, eps)
        f = 0.5 * (f + ft)
        g = 0.5 * (g + gt)
        if record:
            fs.append(f.copy())
            gs.append(g.copy())
    if record:
        return f, g, fs, gs
    return f, g


def plan(C, a, b, f, g, eps):
    """Coupling induced by any potentials: P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps).

    §3.2 / App. E.1: the transport-application identity holds for arbitrary
    (f, g); the a_i, b_j factors follow from E.1's induced marginals.
    """
    C = _f64(C)
    E = (_f64(f)[:, None] + _f64(g)[None, :] - C) / eps
    return _f64(a)[:, None] * _f64(b)[None, :] * np.exp(E)


def marginals(P):
    """Actual marginals r = P 1_m and c = P^T 1_n (§2.2, App. E.1)."""
    P = _f64(P)
    return P.sum(axis=1), P.sum(axis=0)


def marginal_errors(P, a, b):
    """L1 marginal violations (||P 1 - a||_1, ||P^T 1 - b||_1) of a coupling (§2.2)."""
    r, c = marginals(P)
    return float(np.abs(r - _f64(a)).sum()), float(np.abs(c - _f64(b)).sum())


def apply_plan(P, V):
    """Transport-matrix application P V (§3.2, Prop. 3, Algorithm 2's output)."""
    return _f64(P) @ _f64(V)


def apply_plan_t(P, U):
    """Adjoint application P^T U (App. E.1 column form, Algorithm 4's output)."""
    return _f64(P).T @ _f64(U)


def barycentric(P, V):
    """Entropic barycentric projection (P V) / r row-wise (§3.2)."""
    P = _f64(P)
    r = P.sum(axis=1)
    return (P @ _f64(V)) / r[:, None]


def grad_x(X, Y, P):
    """Gradient of sum_ij P_ij ||x_i - y_j||^2 in X with P held fixed: 2 (r * X - P Y).

    §2.2 and App. G.1 ("Gradient", induced marginals): with r = P 1 the
    derivative of each cost term 2 (x_i - y_j) summed against P_ij.
    """
    P = _f64(P)
    r = P.sum(axis=1)
    return 2.0 * (r[:, None] * _f64(X) - P @ _f64(Y))


def dual_value(a, b, f, g):
    """Dual objective <a, f> + <b, g> at a fixed point (§4.1: forward returns potentials and cost)."""
    return float(_f64(a) @ _f64(f) + _f64(b) @ _f64(g))


# --- one-at-a-time evaluators for sampled checks at full problem size --------
# They compute single rows/columns of the same definitions without forming the
# whole n x m cost, so that outputs of very large runs can be checked entry by
# entry. They call the dense functions above on a slice.

def update_f_rows(X_rows, Y, g, b, eps):
    """f-half-step for a subset of rows: the definition of ``update_f`` on C[rows, :]."""
    return update_f(cost_matrix(X_rows, Y), g, b, eps)


def update_g_cols(X, Y_cols, f, a, eps):
    """g-half-step for a subset of columns: the definition of ``update_g`` on C[:, cols]."""
    return update_g(cost_matrix(X, Y_cols), f, a, eps)


def plan_rows(X_rows, Y, a_rows, b, f_rows, g, eps):
    """Rows P[rows, :] of the coupling induced by (f, g)."""
    return plan(cost_matrix(X_rows, Y), a_rows, b, f_rows, g, eps)


def plan_cols(X, Y_cols, a, b_cols, f, g_cols, eps):
    """Columns P[:, cols] of the coupling induced by (f, g)."""
    return plan(cost_matrix(X, Y_cols), a, b_cols, f, g_cols, eps)
