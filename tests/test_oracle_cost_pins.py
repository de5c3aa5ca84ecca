"""Pins of the fp64 cost-matrix oracle (``oracle/costs.py``), CPU only: library
routines (scipy cdist), the reductions the page states (§3.1: squared
Euclidean is the affine cost with alpha = ||x||^2, beta = ||y||^2, Q = 2x,
K = y; cosine is half the squared distance of normalised points) and brute
force over pairs."""

import numpy as np
from scipy.spatial.distance import cdist

import oracle
from oracle import costs

RNG = np.random.default_rng(20260404)


def test_affine_reduces_to_squared_euclidean():
    X = RNG.standard_normal((7, 3))
    Y = RNG.standard_normal((5, 3))
    C = costs.cost_affine((X * X).sum(1), (Y * Y).sum(1), 2.0 * X, Y)
    np.testing.assert_allclose(C, cdist(X, Y, "sqeuclidean"), rtol=1e-12, atol=1e-12)


def test_affine_brute_force():
    al, be = RNG.standard_normal(4), RNG.standard_normal(6)
    Q, K = RNG.standard_normal((4, 5)), RNG.standard_normal((6, 5))
    C = costs.cost_affine(al, be, Q, K)
    for i in range(4):
        for j in range(6):
            assert abs(C[i, j] - (al[i] + be[j] - sum(Q[i, k] * K[j, k] for k in range(5)))) < 1e-12


def test_cosine_matches_scipy_and_half_squared_distance_of_unit_vectors():
    X = RNG.standard_normal((9, 4)) * 3.0
    Y = RNG.standard_normal((6, 4)) + 0.5
    C = costs.cost_cosine(X, Y)
    np.testing.assert_allclose(C, cdist(X, Y, "cosine"), rtol=1e-12, atol=1e-12)
    Xh = X / np.linalg.norm(X, axis=1, keepdims=True)
    Yh = Y / np.linalg.norm(Y, axis=1, keepdims=True)
    np.testing.assert_allclose(C, 0.5 * cdist(Xh, Yh, "sqeuclidean"), rtol=1e-12, atol=1e-12)
    # scale invariance of each point
    np.testing.assert_allclose(costs.cost_cosine(X * 7.0, Y * 0.1), C, rtol=1e-12, atol=1e-12)


def test_cosine_zero_row_costs_one():
    X = np.vstack([np.zeros(3), RNG.standard_normal(3)])
    Y = RNG.standard_normal((4, 3))
    C = costs.cost_cosine(X, Y)
    assert np.all(C[0] == 1.0)


def test_labels_brute_force_and_reductions():
    X = RNG.standard_normal((6, 3))
    Y = RNG.standard_normal((5, 3))
    lx = RNG.integers(0, 4, 6)
    ly = RNG.integers(0, 4, 5)
    W = RNG.uniform(0, 2, (4, 4))
    C = costs.cost_labels(X, Y, lx, ly, W)
    for i in range(6):
        for j in range(5):
            ref = sum((X[i, k] - Y[j, k]) ** 2 for k in range(3)) + W[lx[i], ly[j]]
            assert abs(C[i, j] - ref) < 1e-12
    np.testing.assert_allclose(costs.cost_labels(X, Y, lx, ly, np.zeros((4, 4))),
                               oracle.cost_matrix(X, Y), rtol=1e-12, atol=1e-12)
