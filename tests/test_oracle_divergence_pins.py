"""Pins of the eps-scaling and Sinkhorn-divergence oracle (``oracle/divergence.py``),
CPU only: the schedule's closed form, reduction to the plain iteration,
agreement of the annealed and plain fixed points, the marginal identity at
every eps, and the known properties of the debiased divergence with the
squared-Euclidean cost (zero on identical measures, nonnegative, symmetric,
the large-eps limit ||mean(mu) - mean(nu)||^2, i.e. half the MMD of the
kernel -C, and the small-eps limit W_2^2, exact for sorted points in 1-D)."""

import numpy as np
import pytest

import oracle
from oracle import divergence as D

RNG = np.random.default_rng(20260505)


def _cloud(n, d, shift=0.0, rng=RNG):
    X = rng.standard_normal((n, d)) * 0.6 + shift
    a = rng.uniform(0.3, 1.0, n)
    return X, a / a.sum()


def test_eps_schedule_closed_form():
    assert D.eps_schedule(0.1, 6, 1.0, 0.5) == pytest.approx([1.0, 0.5, 0.25, 0.125, 0.1, 0.1])
    assert D.eps_schedule(0.1, 3, 0.05, 0.5) == [0.1, 0.1, 0.1]
    assert D.eps_schedule(0.1, 3) == [0.1, 0.1, 0.1]


def test_eps_scaling_off_is_the_plain_iteration():
    X, a = _cloud(7, 2)
    Y, b = _cloud(6, 2, 0.4)
    C = oracle.cost_matrix(X, Y)
    f1, g1 = D.sinkhorn_eps_scaling(C, a, b, 0.2, 15, 0.1, 0.5)
    f2, g2 = oracle.sinkhorn(C, a, b, 0.2, 15)
    assert np.array_equal(f1, f2) and np.array_equal(g1, g2)


def test_symmetric_eps_scaling_off_is_the_plain_symmetric_iteration():
    X, a = _cloud(6, 2)
    Y, b = _cloud(8, 2, 0.3)
    C = oracle.cost_matrix(X, Y)
    f1, g1 = D.sinkhorn_eps_scaling(C, a, b, 0.2, 12, 0.0, 0.5, schedule="symmetric")
    f2, g2 = oracle.sinkhorn_symmetric(C, a, b, 0.2, 12)
    assert np.array_equal(f1, f2) and np.array_equal(g1, g2)
    # annealed symmetric and alternating solves share the fixed point
    fs, gs = D.sinkhorn_eps_scaling(C, a, b, 0.2, 4000, 3.0, 0.6, schedule="symmetric")
    fa, ga = oracle.sinkhorn(C, a, b, 0.2, 4000)
    np.testing.assert_allclose(oracle.plan(C, a, b, fs, gs, 0.2), oracle.plan(C, a, b, fa, ga, 0.2),
                               rtol=0, atol=1e-10)


def test_eps_scaling_reaches_the_same_coupling():
    X, a = _cloud(8, 2)
    Y, b = _cloud(9, 2, 0.5)
    C = oracle.cost_matrix(X, Y)
    eps = 0.05
    fa, ga = D.sinkhorn_eps_scaling(C, a, b, eps, 3000, 4.0, 0.7)
    fp, gp = oracle.sinkhorn(C, a, b, eps, 3000)
    Pa = oracle.plan(C, a, b, fa, ga, eps)
    Pp = oracle.plan(C, a, b, fp, gp, eps)
    np.testing.assert_allclose(Pa, Pp, rtol=0, atol=1e-10)


def test_column_marginals_exact_after_every_annealed_iteration():
    X, a = _cloud(6, 3)
    Y, b = _cloud(5, 3, 0.2)
    C = oracle.cost_matrix(X, Y)
    sched = D.eps_schedule(0.1, 5, 2.0, 0.5)
    for k in range(1, 6):
        f, g = D.sinkhorn_eps_scaling(C, a, b, 0.1, k, 2.0, 0.5)
        _, c = oracle.marginals(oracle.plan(C, a, b, f, g, sched[k - 1]))
        np.testing.assert_allclose(c, b, rtol=1e-12)


def test_divergence_of_a_measure_with_itself_is_zero():
    X, a = _cloud(7, 3)
    s = D.sinkhorn_divergence(X, X, a, a, 0.3, 50)[0]
    assert abs(s) < 1e-13


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_divergence_nonnegative_and_symmetric(seed):
    rng = np.random.default_rng(seed)
    X, a = _cloud(9, 2, rng=rng)
    Y, b = _cloud(7, 2, shift=rng.uniform(-1, 1), rng=rng)
    s_xy = D.sinkhorn_divergence(X, Y, a, b, 0.2, 2000)[0]
    s_yx = D.sinkhorn_divergence(Y, X, b, a, 0.2, 2000)[0]
    assert s_xy > 0.0
    assert abs(s_xy - s_yx) <= 1e-9 * abs(s_xy)


def test_large_eps_limit_is_squared_mean_difference():
    X, a = _cloud(8, 3)
    Y, b = _cloud(6, 3, 0.7)
    ref = float(np.sum((a @ X - b @ Y) ** 2))
    s = D.sinkhorn_divergence(X, Y, a, b, 1e4, 50)[0]
    assert abs(s - ref) <= 1e-3 * ref


def test_small_eps_limit_is_w2_in_one_dimension():
    n = 6
    x = np.sort(RNG.standard_normal(n))
    y = np.sort(RNG.standard_normal(n) + 0.8)
    u = np.full(n, 1.0 / n)
    w2 = float(np.mean((x - y) ** 2))
    s = D.sinkhorn_divergence(x[:, None], y[:, None], u, u, 2e-3, 20000, eps_start=2.0, decay=0.9)[0]
    assert abs(s - w2) <= 2e-2 * w2
