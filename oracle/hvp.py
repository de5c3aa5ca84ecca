"""fp64 reference of the streaming Hessian-vector product (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the product path never does.

Source: the page "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
(arXiv 2602.03067), §3.3 "Streaming Hessian-Vector Products" (Thm. 5),
App. F.1-F.3 and App. G.1 ("HVP", induced marginals), App. H.2.3 (parity
protocol). The page's display equations (its eq. 25-31) did not survive, so
this module works the Hessian out from the parts the text keeps, and states
each step:

* T = d^2/dX^2 OT_eps(mu, nu) with Y fixed, and T A its product with a
  direction A (n x d). The gradient is grad_i = 2 sum_j P_ij (x_i - y_j)
  (App. G.1). Differentiating it along A, with
  P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) and dC_ij = 2 (x_i - y_j).A_i,
  splits T A into an explicit part (P moves with C at fixed potentials) and
  an implicit part (the potentials move to keep the marginals):
      T A = E A + (1/eps) R^T w,  H* w = R A.
* Explicit part (App. F.1, F.3: "E A = B1 - (4/eps)(B2 - B3 - B4 + B5)",
  block k = 2 a_k I - (4/eps) sum_j P_kj (x_k - y_j)(x_k - y_j)^T):
      B1 = 2 r * A,            B2 = (r * <x_i, A_i>) x_i,
      B3 = <x_i, A_i> (P Y)_i,  B4 = ((P . A Y^T) 1)_i x_i,
      B5 = (P . A Y^T) Y   (the Hadamard-weighted transport, Algorithm 5),
  with r, c the induced marginals of the coupling (App. G.1).
* Sensitivity matrix (App. G.1 "HVP"): H* = [[diag r, P], [P^T, diag c]],
  singular with the one null vector (1, -1) (App. A: shift of potentials).
* R A = (sum_j P_ij dC_ij, sum_i P_ij dC_ij): the change of the two marginal
  conditions; R^T w = 2 sum_j P_ij (w1_i + w2_j)(x_i - y_j). The implicit
  part (1/eps) R^T H*^+ R is PSD (App. F.2 summary).
* Damped Schur complement (§3.3, App. F.2 step 2): eliminating w1 gives
  S w2 = R2 - P^T (R1 / r) with S = diag c - P^T diag(1/r) P; the page solves
  S_tau = S + tau I by conjugate gradients stopped at relative residual eta,
  then w1 = (R1 - P w2) / r (back-substitution).
* Dense reference (App. H.2.3): H*'s pseudoinverse from an eigendecomposition
  with threshold 1e-10 (read here as relative to the largest |eigenvalue|).

Everything is formed densely: P is materialised, and no term is streamed,
fused or reordered.
"""

from __future__ import annotations

import numpy as np

from .sinkhorn import cost_matrix, plan


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _coupling(X, Y, a, b, f, g, eps):
    return plan(cost_matrix(X, Y), a, b, f, g, eps)


def sensitivity_matrix(P):
    """H* = [[diag r, P], [P^T, diag c]] with the induced marginals r = P 1, c = P^T 1
    (App. G.1 "HVP": built from the current coupling's marginals)."""
    P = _f64(P)
    n, m = P.shape
    H = np.zeros((n + m, n + m))
    H[:n, :n] = np.diag(P.sum(axis=1))
    H[n:, n:] = np.diag(P.sum(axis=0))
    H[:n, n:] = P
    H[n:, :n] = P.T
    return H


def explicit_term(X, Y, P, A, eps):
    """E A = B1 - (4/eps)(B2 - B3 - B4 + B5) (App. F.1, F.3): the derivative of
    the gradient along A with the potentials held fixed."""
    X, Y, P, A = _f64(X), _f64(Y), _f64(P), _f64(A)
    r = P.sum(axis=1)
    xa = np.einsum("ik,ik->i", X, A)
    W = P * (A @ Y.T)                    # P . (A Y^T)
    B1 = 2.0 * r[:, None] * A
    B2 = (r * xa)[:, None] * X
    B3 = xa[:, None] * (P @ Y)
    B4 = W.sum(axis=1)[:, None] * X
    B5 = W @ Y
    return B1 - (4.0 / eps) * (B2 - B3 - B4 + B5)


def sensitivity_rhs(X, Y, P, A):
    """R A = (sum_j P_ij dC_ij, sum_i P_ij dC_ij) with dC_ij = 2 (x_i - y_j).A_i:
    the first-order change of the row and column sums of P at fixed potentials."""
    X, Y, P, A = _f64(X), _f64(Y), _f64(P), _f64(A)
    dC = 2.0 * (np.einsum("ik,ik->i", X, A)[:, None] - A @ Y.T)
    PdC = P * dC
    return PdC.sum(axis=1), PdC.sum(axis=0)


def implicit_apply(X, Y, P, w1, w2):
    """R^T w = 2 sum_j P_ij (w1_i + w2_j)(x_i - y_j) (App. F.2 step 3)."""
    X, Y, P = _f64(X), _f64(Y), _f64(P)
    Wt = P * (_f64(w1)[:, None] + _f64(w2)[None, :])
    return 2.0 * (Wt.sum(axis=1)[:, None] * X - Wt @ Y)


def pinv_eig(H, rcond=1e-10):
    """Moore-Penrose pseudoinverse of a symmetric matrix by eigendecomposition,
    dropping eigenvalues with |lambda| <= rcond * max|lambda| (App. H.2.3)."""
    lam, U = np.linalg.eigh(_f64(H))
    keep = np.abs(lam) > rcond * np.abs(lam).max()
    inv = np.zeros_like(lam)
    inv[keep] = 1.0 / lam[keep]
    return (U * inv) @ U.T


def hvp_dense(X, Y, a, b, f, g, eps, A, rcond=1e-10):
    """Reference T A = E A + (1/eps) R^T H*^+ R A with the eigendecomposition
    pseudoinverse (App. H.2.3's dense reference G_star)."""
    P = _coupling(X, Y, a, b, f, g, eps)
    n = P.shape[0]
    R1, R2 = sensitivity_rhs(X, Y, P, A)
    w = pinv_eig(sensitivity_matrix(P), rcond) @ np.concatenate([R1, R2])
    return explicit_term(X, Y, P, A, eps) + implicit_apply(X, Y, P, w[:n], w[n:]) / eps


def schur_rhs(P, R1, R2):
    """Right side of the Schur system after eliminating w1: R2 - P^T (R1 / r)."""
    P = _f64(P)
    r = P.sum(axis=1)
    return _f64(R2) - P.T @ (_f64(R1) / r)


def conjugate_gradient(apply_op, rhs, iters, tol):
    """Textbook conjugate gradients (Hestenes-Stiefel) from x = 0 for an SPD
    operator. Stops after `iters` iterations, or once ||res|| <= tol ||rhs||
    (tol = 0: always `iters`). Returns (x, iterations run, ||res|| / ||rhs||)."""
    rhs = _f64(rhs)
    x = np.zeros_like(rhs)
    res = rhs.copy()
    p = res.copy()
    rr = float(res @ res)
    bb = rr
    if bb == 0.0:
        return x, 0, 0.0
    k = 0
    while k < iters and rr > (tol * tol) * bb:
        q = apply_op(p)
        alpha = rr / float(p @ q)
        x = x + alpha * p
        res = res - alpha * q
        rr_new = float(res @ res)
        p = res + (rr_new / rr) * p
        rr = rr_new
        k += 1
    return x, k, float(np.sqrt(rr / bb))


def hvp_schur_cg(X, Y, a, b, f, g, eps, A, tau, iters, tol=0.0):
    """Regularised T A (§3.3, App. F.2): S_tau w2 = R2 - P^T (R1 / r) by conjugate
    gradients with S_tau = diag c - P^T diag(1/r) P + tau I, back-substitution
    w1 = (R1 - P w2) / r, then E A + (1/eps) R^T w.

    Returns (G, iterations run, final relative residual)."""
    P = _coupling(X, Y, a, b, f, g, eps)
    r, c = P.sum(axis=1), P.sum(axis=0)
    R1, R2 = sensitivity_rhs(X, Y, P, A)

    def s_tau(v):
        return c * v - P.T @ ((P @ v) / r) + tau * v

    w2, k, rel = conjugate_gradient(s_tau, schur_rhs(P, R1, R2), iters, tol)
    w1 = (R1 - P @ w2) / r
    G = explicit_term(X, Y, P, A, eps) + implicit_apply(X, Y, P, w1, w2) / eps
    return G, k, rel
