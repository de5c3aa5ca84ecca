"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the passage of "FlashSinkhorn: IO-Aware Entropic Optimal
Transport on GPU" (arXiv 2602.03067) or the piece of mathematics that fixes
the expected value. Together they are chosen so that a plausible slip in the
oracle (a dropped log-weight, a sign, a swapped update order, a transposed
operand, a missing factor 2 in the gradient) fails at least one of them:

* marginal identities after each half-step (App. E.1 induced marginals);
* the classic kernel-domain scaling iteration u = a / (K v), v = b / (K^T u),
  an independent textbook formulation of the same alternating schedule;
* closed forms: m = 1, the 2 x 2 uniform problem, the eps -> infinity limit;
* invariances: constant shift of the potentials, common translation of points;
* brute force: exact OT over all permutations for n = m <= 7 and the 1-D
  monotone rearrangement, both within the entropic sandwich [0, eps log n];
* central finite differences of the converged dual value for the gradient;
* library routines (scipy cdist, scipy logsumexp) for the building blocks.

No GPU is used here.
"""

import itertools
import math

import numpy as np
import pytest
from scipy.spatial.distance import cdist
from scipy.special import logsumexp as sp_lse

import oracle

RNG = np.random.default_rng(20260202)


def _problem(n, m, d, uniform=False, rng=RNG):
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((m, d)) * 0.7 + 0.3
    if uniform:
        a = np.full(n, 1.0 / n)
        b = np.full(m, 1.0 / m)
    else:
        a = rng.uniform(0.2, 1.0, n)
        a /= a.sum()
        b = rng.uniform(0.2, 1.0, m)
        b /= b.sum()
    return X, Y, a, b


def _converge(C, a, b, eps, tol=1e-13, max_iter=200000):
    f = np.zeros(C.shape[0])
    g = np.zeros(C.shape[1])
    for it in range(max_iter):
        f = oracle.update_f(C, g, b, eps)
        g = oracle.update_g(C, f, a, eps)
        if it % 10 == 0:
            er, _ = oracle.marginal_errors(oracle.plan(C, a, b, f, g, eps), a, b)
            if er < tol:
                break
    return f, g


# --- building blocks against library routines ---------------------------------

def test_cost_matrix_matches_scipy_cdist():
    """Cost = squared Euclidean distance (§3.1 'Scope of cost structure', App. H.2)."""
    X, Y, _, _ = _problem(17, 11, 5)
    C = oracle.cost_matrix(X, Y)
    np.testing.assert_allclose(C, cdist(X, Y, "sqeuclidean"), rtol=1e-13, atol=1e-13)
    # blocked evaluation must not change values
    np.testing.assert_array_equal(oracle.cost_matrix(X, Y, block_elems=7), C)
    # hand-worked example: (0,0) vs (3,4) -> 25; (1,2) vs (1,2) -> 0
    C2 = oracle.cost_matrix([[0.0, 0.0], [1.0, 2.0]], [[3.0, 4.0], [1.0, 2.0]])
    np.testing.assert_array_equal(C2, [[25.0, 5.0], [8.0, 0.0]])


def test_sqnorms_matches_linalg():
    X, _, _, _ = _problem(9, 3, 7)
    np.testing.assert_allclose(oracle.sqnorms(X), np.linalg.norm(X, axis=1) ** 2, rtol=1e-14)


def test_logsumexp_matches_scipy_and_merges():
    """LSE value and the online-merge property (App. D.3; merge of partial statistics)."""
    Z = RNG.standard_normal((6, 50)) * 30
    np.testing.assert_allclose(oracle.logsumexp(Z, 1), sp_lse(Z, axis=1), rtol=1e-14)
    np.testing.assert_allclose(oracle.logsumexp(Z, 0), sp_lse(Z, axis=0), rtol=1e-14)
    # LSE over a union equals LSE of the per-part LSEs, for any partition.
    parts = [Z[:, :7], Z[:, 7:31], Z[:, 31:]]
    merged = oracle.logsumexp(np.stack([oracle.logsumexp(p, 1) for p in parts], 1), 1)
    np.testing.assert_allclose(merged, oracle.logsumexp(Z, 1), rtol=1e-14)


# --- half-step identities ------------------------------------------------------

@pytest.mark.parametrize("n,m,d,eps", [(13, 9, 3, 0.3), (5, 21, 1, 0.05), (30, 30, 8, 1.0)])
def test_marginal_identity_after_each_half_step(n, m, d, eps):
    """App. E.1: after an f half-step the coupling's row sums equal a exactly,
    after a g half-step its column sums equal b exactly. Non-uniform weights
    and n != m make a dropped log-weight, a sign slip or a transposed cost fail."""
    X, Y, a, b = _problem(n, m, d)
    C = oracle.cost_matrix(X, Y)
    g = RNG.standard_normal(m)
    f = oracle.update_f(C, g, b, eps)
    r, _ = oracle.marginals(oracle.plan(C, a, b, f, g, eps))
    np.testing.assert_allclose(r, a, rtol=1e-11, atol=0)
    g2 = oracle.update_g(C, f, a, eps)
    _, c = oracle.marginals(oracle.plan(C, a, b, f, g2, eps))
    np.testing.assert_allclose(c, b, rtol=1e-11, atol=0)


def test_induced_row_marginal_formula():
    """App. E.1: r = a * exp((f - f+)/eps) where f+ is the next f half-step."""
    X, Y, a, b = _problem(12, 8, 4)
    C = oracle.cost_matrix(X, Y)
    eps = 0.2
    f = RNG.standard_normal(12) * 0.1
    g = RNG.standard_normal(8) * 0.1
    r, _ = oracle.marginals(oracle.plan(C, a, b, f, g, eps))
    fplus = oracle.update_f(C, g, b, eps)
    np.testing.assert_allclose(r, a * np.exp((f - fplus) / eps), rtol=1e-12)


def test_matches_kernel_domain_scaling_iteration():
    """The textbook Sinkhorn scaling iteration (K = exp(-C/eps), u = a/(K v),
    v = b/(K^T u), from v = b) is the same alternating schedule written on
    the scalings u = a exp(f/eps), v = b exp(g/eps). It shares no code with
    the log-domain oracle and pins order, signs and weight placement."""
    X, Y, a, b = _problem(10, 14, 3)
    eps = 0.5
    C = oracle.cost_matrix(X, Y)
    K = np.exp(-C / eps)
    u = np.ones(10)
    v = b.copy()
    f, g = np.zeros(10), np.zeros(14)
    for _ in range(25):
        u = a / (K @ v)
        v = b / (K.T @ u)
        f = oracle.update_f(C, g, b, eps)
        g = oracle.update_g(C, f, a, eps)
    np.testing.assert_allclose(f, eps * np.log(u / a), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g, eps * np.log(v / b), rtol=1e-10, atol=1e-12)
    f2, g2 = oracle.sinkhorn(C, a, b, eps, 25)
    np.testing.assert_array_equal(f2, f)
    np.testing.assert_array_equal(g2, g)


# --- closed forms ----------------------------------------------------------------

def test_single_target_point_closed_form():
    """m = 1 (b = [1]): f_i = C_i1 - g_1, then g_1 = -eps log(sum a) = 0; the
    coupling is a, and P V = a V_1^T (every mass goes to the one target)."""
    X, Y, a, _ = _problem(9, 1, 4)
    b = np.array([1.0])
    C = oracle.cost_matrix(X, Y)
    f, g = oracle.sinkhorn(C, a, b, 0.1, 1)
    np.testing.assert_allclose(f, C[:, 0], rtol=1e-13)
    assert abs(g[0]) < 1e-13
    f3, g3 = oracle.sinkhorn(C, a, b, 0.1, 3)
    np.testing.assert_allclose(f3, f, rtol=1e-13)
    P = oracle.plan(C, a, b, f, g, 0.1)
    np.testing.assert_allclose(P[:, 0], a, rtol=1e-12)
    V = RNG.standard_normal((1, 5))
    np.testing.assert_allclose(oracle.apply_plan(P, V), a[:, None] * V[0][None, :], rtol=1e-12)


@pytest.mark.parametrize("eps", [0.5, 0.2, 0.1])
def test_two_by_two_closed_form(eps):
    """Uniform 2 x 2: P = [[p, 1/2-p], [1/2-p, p]] with P11 P22 / (P12 P21) =
    exp((C12 + C21 - C11 - C22)/eps), i.e. p / (1/2 - p) = exp(Delta / (2 eps))."""
    X = np.array([[0.0, 0.0], [1.0, 0.5]])
    Y = np.array([[0.2, 0.1], [0.9, 0.9]])
    a = b = np.array([0.5, 0.5])
    C = oracle.cost_matrix(X, Y)
    f, g = _converge(C, a, b, eps)
    P = oracle.plan(C, a, b, f, g, eps)
    delta = C[0, 1] + C[1, 0] - C[0, 0] - C[1, 1]
    e = math.exp(delta / (2 * eps))
    p = 0.5 * e / (1.0 + e)
    np.testing.assert_allclose(P, [[p, 0.5 - p], [0.5 - p, p]], rtol=1e-9, atol=1e-10)


def test_large_eps_limit_is_product_coupling():
    """eps -> infinity: the entropic term dominates and P -> a b^T."""
    X, Y, a, b = _problem(8, 6, 3)
    C = oracle.cost_matrix(X, Y)
    f, g = oracle.sinkhorn(C, a, b, 1e7, 5)
    P = oracle.plan(C, a, b, f, g, 1e7)
    np.testing.assert_allclose(P, np.outer(a, b), rtol=1e-6)


# --- invariances -------------------------------------------------------------------

def test_constant_shift_of_potentials():
    """Starting from g0 + c gives (f - c, g + c) at every iteration with the
    same coupling: the iteration only sees f_i + g_j."""
    X, Y, a, b = _problem(11, 7, 2)
    C = oracle.cost_matrix(X, Y)
    eps = 0.1
    g0 = RNG.standard_normal(7) * 0.3
    c = 0.737
    f1, g1, fs1, gs1 = oracle.sinkhorn(C, a, b, eps, 12, g0=g0, record=True)
    f2, g2, fs2, gs2 = oracle.sinkhorn(C, a, b, eps, 12, g0=g0 + c, record=True)
    for t in range(12):
        np.testing.assert_allclose(fs2[t], fs1[t] - c, atol=1e-12)
        np.testing.assert_allclose(gs2[t], gs1[t] + c, atol=1e-12)
    np.testing.assert_allclose(oracle.plan(C, a, b, f2, g2, eps),
                               oracle.plan(C, a, b, f1, g1, eps), rtol=1e-10)


def test_common_translation_leaves_potentials_unchanged():
    """The squared-Euclidean cost depends only on x_i - y_j."""
    X, Y, a, b = _problem(9, 12, 6)
    shift = RNG.standard_normal(6) * 5
    f1, g1 = oracle.sinkhorn(oracle.cost_matrix(X, Y), a, b, 0.1, 20)
    f2, g2 = oracle.sinkhorn(oracle.cost_matrix(X + shift, Y + shift), a, b, 0.1, 20)
    np.testing.assert_allclose(f2, f1, atol=1e-10)
    np.testing.assert_allclose(g2, g1, atol=1e-10)


def test_iterations_compose():
    """k iterations then k' more from the result equal k + k' iterations (warm start)."""
    X, Y, a, b = _problem(9, 10, 3)
    C = oracle.cost_matrix(X, Y)
    f, g = oracle.sinkhorn(C, a, b, 0.1, 7)
    f2, g2 = oracle.sinkhorn(C, a, b, 0.1, 5, f0=f, g0=g)
    f3, g3 = oracle.sinkhorn(C, a, b, 0.1, 12)
    np.testing.assert_array_equal(f2, f3)
    np.testing.assert_array_equal(g2, g3)


# --- brute force -----------------------------------------------------------------------

@pytest.mark.parametrize("n,seed", [(4, 1), (5, 2), (6, 3), (7, 4)])
def test_bruteforce_assignment_sandwich(n, seed):
    """Uniform weights, n = m: OT_0 is attained at a permutation (Birkhoff), so
    OT_0 = min_sigma (1/n) sum_i C_{i sigma(i)}. The converged entropic plan
    obeys 0 <= <P, C> - OT_0 <= eps log n (KL(P|ab^T) >= 0 and KL of the
    optimal permutation = log n); with a unique optimum the row argmax of P
    recovers sigma* once eps is small against the optimality gap."""
    rng = np.random.default_rng(seed)
    X = rng.uniform(0, 1, (n, 2))
    Y = rng.uniform(0, 1, (n, 2))
    a = b = np.full(n, 1.0 / n)
    C = oracle.cost_matrix(X, Y)
    costs = {p: C[np.arange(n), p].mean() for p in itertools.permutations(range(n))}
    best = min(costs, key=costs.get)
    ot0 = costs[best]
    gap = sorted(costs.values())[1] - ot0
    for eps in (0.05, 0.02, 0.01):
        f, g = _converge(C, a, b, eps, tol=1e-11)
        P = oracle.plan(C, a, b, f, g, eps)
        primal = float((P * C).sum())
        assert -1e-9 <= primal - ot0 <= eps * math.log(n) + 1e-9
        if gap > 8 * eps * math.log(n):
            assert tuple(np.argmax(P, axis=1)) == best


def test_one_dimensional_monotone_rearrangement():
    """d = 1, uniform weights: OT_0 = (1/n) sum (x_(i) - y_(i))^2 by sorting
    (monotone rearrangement); the converged entropic cost sits in the sandwich."""
    rng = np.random.default_rng(7)
    n = 200
    x = rng.uniform(0, 1, (n, 1))
    y = rng.normal(0.5, 0.2, (n, 1))
    ot0 = float(np.mean((np.sort(x[:, 0]) - np.sort(y[:, 0])) ** 2))
    a = b = np.full(n, 1.0 / n)
    C = oracle.cost_matrix(x, y)
    eps = 0.002
    f, g = _converge(C, a, b, eps, tol=1e-10, max_iter=50000)
    P = oracle.plan(C, a, b, f, g, eps)
    primal = float((P * C).sum())
    assert -1e-9 <= primal - ot0 <= eps * math.log(n)


# --- dual value, gradient, transport application ------------------------------------

def test_dual_equals_primal_at_convergence():
    """Entropic strong duality: <a,f> + <b,g> = <P,C> + eps KL(P | a b^T) at the fixed point."""
    X, Y, a, b = _problem(10, 12, 3)
    C = oracle.cost_matrix(X, Y)
    eps = 0.3
    f, g = _converge(C, a, b, eps)
    P = oracle.plan(C, a, b, f, g, eps)
    kl = float((P * np.log(P / np.outer(a, b))).sum())
    assert abs(oracle.dual_value(a, b, f, g) - ((P * C).sum() + eps * kl)) < 1e-11


def test_gradient_matches_finite_differences():
    """§2.2 / App. G.1: d/dX of the converged value <a,f> + <b,g> equals
    2 (r * X - P Y) (envelope theorem; r = a at the fixed point)."""
    X, Y, a, b = _problem(5, 4, 2)
    eps = 0.5

    def value(Xv):
        C = oracle.cost_matrix(Xv, Y)
        f, g = _converge(C, a, b, eps, tol=1e-14)
        return oracle.dual_value(a, b, f, g)

    C = oracle.cost_matrix(X, Y)
    f, g = _converge(C, a, b, eps, tol=1e-14)
    G = oracle.grad_x(X, Y, oracle.plan(C, a, b, f, g, eps))
    h = 1e-5
    fd = np.zeros_like(X)
    for i in range(X.shape[0]):
        for k in range(X.shape[1]):
            Xp = X.copy()
            Xm = X.copy()
            Xp[i, k] += h
            Xm[i, k] -= h
            fd[i, k] = (value(Xp) - value(Xm)) / (2 * h)
    np.testing.assert_allclose(G, fd, rtol=1e-6, atol=1e-8)


def test_apply_plan_identities():
    """P 1 = r (= a right after an f half-step); P^T 1 = c; P^T U = (U^T P)^T;
    the barycentric projection of a permutation coupling returns the matched points."""
    X, Y, a, b = _problem(8, 5, 3)
    C = oracle.cost_matrix(X, Y)
    eps = 0.25
    g = RNG.standard_normal(5) * 0.2
    f = oracle.update_f(C, g, b, eps)
    P = oracle.plan(C, a, b, f, g, eps)
    np.testing.assert_allclose(oracle.apply_plan(P, np.ones((5, 1)))[:, 0], a, rtol=1e-12)
    _, c = oracle.marginals(P)
    np.testing.assert_allclose(oracle.apply_plan_t(P, np.ones((8, 1)))[:, 0], c, rtol=1e-12)
    U = RNG.standard_normal((8, 3))
    np.testing.assert_allclose(oracle.apply_plan_t(P, U), (U.T @ P).T, rtol=1e-12)
    # permutation coupling
    perm = np.array([2, 0, 1])
    Pp = np.zeros((3, 3))
    Pp[np.arange(3), perm] = 1.0 / 3
    V = RNG.standard_normal((3, 2))
    np.testing.assert_allclose(oracle.barycentric(Pp, V), V[perm], rtol=1e-14)


def test_marginals_and_errors_worked_by_hand():
    """A 2 x 2 coupling worked by hand: row sums (0.3, 0.7), column sums
    (0.4, 0.6); against a = (0.25, 0.75), b = (0.5, 0.5) the L1 errors are
    0.05 + 0.05 = 0.1 and 0.1 + 0.1 = 0.2 (rows and columns not swapped)."""
    P = np.array([[0.1, 0.2], [0.3, 0.4]])
    r, c = oracle.marginals(P)
    np.testing.assert_allclose(r, [0.3, 0.7], rtol=0, atol=1e-15)
    np.testing.assert_allclose(c, [0.4, 0.6], rtol=0, atol=1e-15)
    er, ec = oracle.marginal_errors(P, np.array([0.25, 0.75]), np.array([0.5, 0.5]))
    assert abs(er - 0.1) < 1e-15 and abs(ec - 0.2) < 1e-15


def test_row_and_column_evaluators_agree_with_dense():
    """The one-at-a-time evaluators are the dense definitions on a slice."""
    X, Y, a, b = _problem(20, 15, 4)
    C = oracle.cost_matrix(X, Y)
    eps = 0.15
    g = RNG.standard_normal(15) * 0.1
    f = oracle.update_f(C, g, b, eps)
    rows = np.array([0, 7, 19])
    np.testing.assert_allclose(oracle.update_f_rows(X[rows], Y, g, b, eps), f[rows], rtol=1e-14)
    g2 = oracle.update_g(C, f, a, eps)
    cols = np.array([1, 14])
    np.testing.assert_allclose(oracle.update_g_cols(X, Y[cols], f, a, eps), g2[cols], rtol=1e-14)
    P = oracle.plan(C, a, b, f, g2, eps)
    np.testing.assert_allclose(oracle.plan_rows(X[rows], Y, a[rows], b, f[rows], g2, eps), P[rows], rtol=1e-13)
    np.testing.assert_allclose(oracle.plan_cols(X, Y[cols], a, b[cols], f, g2[cols], eps), P[:, cols], rtol=1e-13)


def test_dimension_zero_and_single_point():
    """Degenerate shapes: d = 0 (all costs 0) gives f_i = -eps log(sum b) - g-part,
    and n = m = 1 couples the single pair with mass a_1 b_1-consistent potentials."""
    X = np.zeros((4, 0))
    Y = np.zeros((3, 0))
    C = oracle.cost_matrix(X, Y)
    assert C.shape == (4, 3) and np.all(C == 0)
    a = np.full(4, 0.25)
    b = np.full(3, 1.0 / 3)
    f, g = oracle.sinkhorn(C, a, b, 0.1, 3)
    np.testing.assert_allclose(oracle.plan(C, a, b, f, g, 0.1), np.outer(a, b), rtol=1e-12)
    C1 = oracle.cost_matrix([[1.0, 2.0]], [[0.0, 0.0]])
    f1, g1 = oracle.sinkhorn(C1, [1.0], [1.0], 0.1, 2)
    assert abs(f1[0] + g1[0] - C1[0, 0]) < 1e-13


# --- symmetric (averaged) schedule ---------------------------------------------------

def test_symmetric_schedule_matches_scaling_geometric_mean():
    """The averaged log-domain update is the geometric mean of the old scaling
    and the textbook scaling update, both taken from the old iterate:
    u <- sqrt(u * a / (K v)), v <- sqrt(v * b / (K^T u)) with u = a exp(f/eps),
    v = b exp(g/eps), K = exp(-C/eps). Written on the scalings, it shares no
    code with the log-domain oracle and pins the averaging, the use of the old
    iterate in both half-steps, and the weights."""
    X, Y, a, b = _problem(9, 12, 3)
    eps = 0.5
    C = oracle.cost_matrix(X, Y)
    K = np.exp(-C / eps)
    u, v = a.copy(), b.copy()
    for _ in range(30):
        u, v = np.sqrt(u * a / (K @ v)), np.sqrt(v * b / (K.T @ u))
    f, g = oracle.sinkhorn_symmetric(C, a, b, eps, 30)
    np.testing.assert_allclose(f, eps * np.log(u / a), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g, eps * np.log(v / b), rtol=1e-10, atol=1e-12)


def test_symmetric_and_alternating_share_the_fixed_point():
    """Both schedules converge to the Sinkhorn fixed point: the coupling has
    marginals a and b, and the two converged couplings coincide (the potentials
    themselves may differ by the constant mode f + k, g - k)."""
    X, Y, a, b = _problem(11, 8, 2)
    eps = 0.4
    C = oracle.cost_matrix(X, Y)
    fa, ga = oracle.sinkhorn(C, a, b, eps, 4000)
    fs, gs = oracle.sinkhorn_symmetric(C, a, b, eps, 4000)
    Pa = oracle.plan(C, a, b, fa, ga, eps)
    Ps = oracle.plan(C, a, b, fs, gs, eps)
    r, c = oracle.marginals(Ps)
    np.testing.assert_allclose(r, a, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(c, b, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(Ps, Pa, rtol=1e-8, atol=1e-13)


def test_symmetric_schedule_constant_shift():
    """Starting from (f0 + k, g0 - k) shifts every iterate by (+k, -k) and leaves
    the coupling unchanged: T_f(g - k) = T_f(g) + k and T_g(f + k) = T_g(f) - k."""
    X, Y, a, b = _problem(7, 9, 3)
    eps = 0.3
    C = oracle.cost_matrix(X, Y)
    f0 = RNG.standard_normal(7) * 0.2
    g0 = RNG.standard_normal(9) * 0.2
    k = 0.37
    f1, g1 = oracle.sinkhorn_symmetric(C, a, b, eps, 6, f0, g0)
    f2, g2 = oracle.sinkhorn_symmetric(C, a, b, eps, 6, f0 + k, g0 - k)
    np.testing.assert_allclose(f2, f1 + k, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g2, g1 - k, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.plan(C, a, b, f2, g2, eps), oracle.plan(C, a, b, f1, g1, eps),
                               rtol=1e-11)
