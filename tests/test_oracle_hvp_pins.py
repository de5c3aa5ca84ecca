"""Pins of the fp64 Hessian-vector-product oracle (``oracle/hvp.py``), CPU only.

The page's HVP equations (§3.3 Thm. 5, App. F) are garbled, so the oracle's
formulas are a derivation; these tests tie that derivation to things that do
not depend on it:

* central finite differences of the gradient at converged potentials (the
  definition of the Hessian: catches a dropped term, a wrong sign or a
  transposed operand anywhere in E A, R A, R^T w or the solve);
* the single-target closed form (m = 1: OT = sum_i a_i ||x_i - y||^2 minus a
  constant, so T A = 2 a * A exactly; the explicit part alone is far off);
* symmetry of the Hessian, PSD-ness of the implicit part (App. F.2 summary),
  the null vector of H* (App. F / App. A shift invariance);
* App. F.3's block form of E (per-point outer products) against the
  B1..B5 assembly;
* library routines for the linear algebra (numpy pinv, a dense solve of the
  damped Schur system) against the eigendecomposition pseudoinverse and the
  conjugate-gradient solver;
* invariance of T A under a common translation of both clouds.
"""

import numpy as np
import pytest

import oracle
from oracle import hvp as H

RNG = np.random.default_rng(20260303)


def _problem(n, m, d, rng=RNG):
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((m, d)) * 0.7 + 0.3
    a = rng.uniform(0.2, 1.0, n)
    a /= a.sum()
    b = rng.uniform(0.2, 1.0, m)
    b /= b.sum()
    return X, Y, a, b


def _converge(X, Y, a, b, eps, tol=1e-14, max_iter=200000):
    C = oracle.cost_matrix(X, Y)
    f = np.zeros(len(a))
    g = np.zeros(len(b))
    for _ in range(max_iter):
        f = oracle.update_f(C, g, b, eps)
        g = oracle.update_g(C, f, a, eps)
        er, _ = oracle.marginal_errors(oracle.plan(C, a, b, f, g, eps), a, b)
        if er < tol:
            break
    return f, g


def _grad(X, Y, a, b, eps):
    f, g = _converge(X, Y, a, b, eps)
    return oracle.grad_x(X, Y, oracle.plan(oracle.cost_matrix(X, Y), a, b, f, g, eps))


def _rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("n,m,d,eps", [(6, 5, 2, 0.5), (5, 7, 3, 0.2)])
def test_hvp_matches_finite_difference_of_gradient(n, m, d, eps):
    """T A = d/dh grad(X + h A) at h = 0, the gradient taken at converged
    potentials (envelope theorem, pinned by the gradient's own test)."""
    X, Y, a, b = _problem(n, m, d)
    A = RNG.standard_normal((n, d))
    f, g = _converge(X, Y, a, b, eps)
    G = H.hvp_dense(X, Y, a, b, f, g, eps, A)
    h = 1e-5
    fd = (_grad(X + h * A, Y, a, b, eps) - _grad(X - h * A, Y, a, b, eps)) / (2 * h)
    assert _rel(G, fd) < 1e-7


def test_single_target_closed_form():
    """m = 1: every x_i sends its whole mass to y, OT_eps = sum_i a_i ||x_i - y||^2
    (the entropy term is constant), hence T A = 2 a * A. The explicit part alone
    is far from it: the implicit part must cancel the rest."""
    X, _, a, _ = _problem(7, 1, 3)
    Y = RNG.standard_normal((1, 3))
    b = np.ones(1)
    eps = 0.3
    A = RNG.standard_normal(X.shape)
    f, g = _converge(X, Y, a, b, eps)
    G = H.hvp_dense(X, Y, a, b, f, g, eps, A)
    np.testing.assert_allclose(G, 2.0 * a[:, None] * A, rtol=0, atol=1e-11)
    P = oracle.plan(oracle.cost_matrix(X, Y), a, b, f, g, eps)
    assert np.abs(H.explicit_term(X, Y, P, A, eps) - 2.0 * a[:, None] * A).max() > 1e-2


def test_hessian_is_symmetric():
    X, Y, a, b = _problem(8, 6, 3)
    eps = 0.4
    f, g = _converge(X, Y, a, b, eps)
    A = RNG.standard_normal(X.shape)
    B = RNG.standard_normal(X.shape)
    lhs = float(np.sum(B * H.hvp_dense(X, Y, a, b, f, g, eps, A)))
    rhs = float(np.sum(A * H.hvp_dense(X, Y, a, b, f, g, eps, B)))
    assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1.0)


def test_implicit_part_is_psd_and_h_has_the_shift_null_vector():
    """App. F.2 summary: (1/eps) R^T H^+ R is PSD. H* (1, -1) = 0 (a constant
    shift of f against g leaves P unchanged), and R A has no component along
    that vector, so the system H* w = R A is consistent."""
    X, Y, a, b = _problem(9, 7, 2)
    eps = 0.25
    f, g = _converge(X, Y, a, b, eps)
    P = oracle.plan(oracle.cost_matrix(X, Y), a, b, f, g, eps)
    Hs = H.sensitivity_matrix(P)
    null = np.concatenate([np.ones(9), -np.ones(7)])
    assert np.abs(Hs @ null).max() < 1e-15
    lam = np.linalg.eigvalsh(Hs)
    assert lam[0] > -1e-14 and np.sum(np.abs(lam) < 1e-12) == 1
    Hp = H.pinv_eig(Hs)
    for _ in range(5):
        A = RNG.standard_normal(X.shape)
        R1, R2 = H.sensitivity_rhs(X, Y, P, A)
        assert abs(R1.sum() - R2.sum()) < 1e-14
        w = Hp @ np.concatenate([R1, R2])
        imp = H.implicit_apply(X, Y, P, w[:9], w[9:]) / eps
        assert float(np.sum(A * imp)) >= -1e-14


def test_explicit_term_equals_block_outer_product_form():
    """App. F.3: E is block-diagonal with blocks
    2 r_k I - (4/eps) sum_j P_kj (x_k - y_j)(x_k - y_j)^T (induced r)."""
    X, Y, a, b = _problem(5, 6, 3)
    eps = 0.35
    f, g = _converge(X, Y, a, b, eps, tol=1e-6)  # any potentials: r is induced
    P = oracle.plan(oracle.cost_matrix(X, Y), a, b, f, g, eps)
    A = RNG.standard_normal(X.shape)
    ref = np.zeros_like(A)
    for k in range(5):
        blk = 2.0 * P[k].sum() * np.eye(3)
        for j in range(6):
            u = X[k] - Y[j]
            blk -= (4.0 / eps) * P[k, j] * np.outer(u, u)
        ref[k] = blk @ A[k]
    np.testing.assert_allclose(H.explicit_term(X, Y, P, A, eps), ref, rtol=1e-13, atol=1e-13)


def test_pinv_eig_matches_numpy_pinv():
    X, Y, a, b = _problem(6, 4, 2)
    f, g = _converge(X, Y, a, b, 0.5)
    Hs = H.sensitivity_matrix(oracle.plan(oracle.cost_matrix(X, Y), a, b, f, g, 0.5))
    np.testing.assert_allclose(H.pinv_eig(Hs), np.linalg.pinv(Hs, rcond=1e-10, hermitian=True),
                               rtol=1e-9, atol=1e-9)


def test_conjugate_gradient_matches_dense_solve():
    """The CG solver on S_tau reaches the dense solution np.linalg.solve(S_tau, rhs),
    and with tau -> 0 the regularised HVP reaches the pseudoinverse reference."""
    X, Y, a, b = _problem(10, 8, 2)
    eps = 0.3
    f, g = _converge(X, Y, a, b, eps)
    P = oracle.plan(oracle.cost_matrix(X, Y), a, b, f, g, eps)
    r, c = P.sum(axis=1), P.sum(axis=0)
    A = RNG.standard_normal(X.shape)
    R1, R2 = H.sensitivity_rhs(X, Y, P, A)
    rhs = H.schur_rhs(P, R1, R2)
    tau = 1e-3
    S = np.diag(c) - P.T @ np.diag(1.0 / r) @ P + tau * np.eye(8)
    x, k, rel = H.conjugate_gradient(lambda v: S @ v, rhs, 100, 1e-13)
    np.testing.assert_allclose(x, np.linalg.solve(S, rhs), rtol=1e-9, atol=1e-12)
    assert rel <= 1e-13 and k <= 100
    G0, _, _ = H.hvp_schur_cg(X, Y, a, b, f, g, eps, A, tau=0.0, iters=200, tol=1e-13)
    assert _rel(G0, H.hvp_dense(X, Y, a, b, f, g, eps, A)) < 1e-9
    # the damped solution moves away from it as tau grows (the page's bias floor)
    G1, _, _ = H.hvp_schur_cg(X, Y, a, b, f, g, eps, A, tau=1e-2, iters=200, tol=1e-13)
    assert _rel(G1, G0) > 1e-4


def test_cg_fixed_iterations_and_zero_rhs():
    X, Y, a, b = _problem(6, 6, 2)
    f, g = _converge(X, Y, a, b, 0.5)
    A = RNG.standard_normal(X.shape)
    _, k, _ = H.hvp_schur_cg(X, Y, a, b, f, g, 0.5, A, tau=1e-5, iters=3, tol=0.0)
    assert k == 3
    x, k, rel = H.conjugate_gradient(lambda v: v, np.zeros(4), 10, 0.0)
    assert k == 0 and rel == 0.0 and not x.any()


def test_common_translation_leaves_hvp_unchanged():
    X, Y, a, b = _problem(6, 5, 3)
    eps = 0.4
    A = RNG.standard_normal(X.shape)
    f, g = _converge(X, Y, a, b, eps)
    G = H.hvp_dense(X, Y, a, b, f, g, eps, A)
    t = np.array([0.7, -1.3, 0.4])
    # a common shift leaves every C_ij, hence the potentials and P, unchanged
    Gt = H.hvp_dense(X + t, Y + t, a, b, f, g, eps, A)
    assert _rel(Gt, G) < 1e-10
