"""GPU parity of the affine, cosine and label-augmented costs (§3.1 "Scope of
cost structure", §4.2) against the fp64 oracle.

The GPU solves each cost as an affine problem (OT_COST_AFFINE), with the
cosine and label features built on the device by ot_prep_cosine /
ot_prep_labels; the oracle forms the cost matrix from its plain definition
(``oracle.costs``) on the original seeded inputs and runs its own Sinkhorn
iteration. Tolerances as for the squared-Euclidean cost: 1e-4 on the
potentials for fp32 features (2e-2 for bf16), 1e-4 relative on P V.
"""

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_amd as ssa
import workloads
from oracle import costs
from gpu_util import DEV, host64, say, zeros

pytestmark = pytest.mark.gpu

POT_TOL = {"f32": 1e-4, "bf16": 2e-2}
PV_TOL = 1e-4


def _t(arr, dtype="f32"):
    t = torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _w64(t):
    return host64(t) if isinstance(t, torch.Tensor) else np.asarray(t, dtype=np.float64)


AFFINE_CASES = [
    # n, m, d, dtype, eps, iters: resident split (d <= 64, d <= 128), tiled wide
    # pass (d > 128), bf16 features
    (333, 517, 16, "f32", 0.1, 30),
    (300, 260, 100, "f32", 0.05, 30),
    (150, 210, 300, "f32", 0.1, 20),
    (260, 300, 64, "bf16", 0.1, 30),
]


@pytest.mark.parametrize("n,m,d,dtype,eps,T", AFFINE_CASES)
def test_affine_cost_solve_and_apply(n, m, d, dtype, eps, T):
    say(f"affine n={n} m={m} d={d} {dtype} eps={eps} T={T}")
    inp = workloads.affine_inputs(n, m, d, seed=n + 3 * m + d)
    Q = _t(inp["Q"], dtype)
    K = _t(inp["K"], dtype)
    al, be = _t(inp["alpha"]), _t(inp["beta"])
    a, b = _t(inp["a"]), _t(inp["b"])
    prob = ssa.problem(Q, K, eps, a, b, x_sqn=al, y_sqn=be, affine=True)
    f, g = zeros(n), zeros(m)
    info = ssa.ot_solve(prob, f, g, T)
    torch.cuda.synchronize()
    a64, b64 = inp["a"].astype(np.float64), inp["b"].astype(np.float64)
    C = costs.cost_affine(inp["alpha"], inp["beta"], host64(Q), host64(K))
    f_ref, g_ref = oracle.sinkhorn(C, a64, b64, eps, T)
    df = np.abs(host64(f) - f_ref).max()
    dg = np.abs(host64(g) - g_ref).max()
    say(f"  max|df|={df:.2e} max|dg|={dg:.2e}")
    assert df <= POT_TOL[dtype] and dg <= POT_TOL[dtype]
    assert not info["nonfinite"]
    # P V of the oracle's potentials (rounded to fp32) under the affine cost
    f32, g32 = f_ref.astype(np.float32), g_ref.astype(np.float32)
    V = np.random.default_rng(d).standard_normal((m, 40)).astype(np.float32)
    pv = ssa.ot_apply_plan(prob, _t(f32), _t(g32), _t(V))
    torch.cuda.synchronize()
    P = oracle.plan(C, a64, b64, f32.astype(np.float64), g32.astype(np.float64), eps)
    ref = oracle.apply_plan(P, V.astype(np.float64))
    err = np.linalg.norm(host64(pv) - ref) / np.linalg.norm(ref)
    say(f"  P V rel err {err:.2e}")
    assert err <= (PV_TOL if dtype == "f32" else 1e-3)


@pytest.mark.parametrize("n,m,d,dtype", [(333, 517, 16, "f32"), (300, 260, 96, "f32"),
                                         (200, 150, 64, "bf16")])
def test_cosine_cost_solve(n, m, d, dtype):
    say(f"cosine n={n} m={m} d={d} {dtype}")
    data = workloads.make("c3_d16_f32", n=n, m=m, d=d)
    X = _t(data["X"], dtype)
    Y = _t(data["Y"], dtype)
    a, b = _t(data["a"]), _t(data["b"])
    eps, T = 0.05, 40
    Xh, hx = ssa.ot_prep_cosine(X)
    Yh, hy = ssa.ot_prep_cosine(Y)
    prob = ssa.problem(Xh, Yh, eps, a, b, x_sqn=hx, y_sqn=hy, affine=True)
    f, g = zeros(n), zeros(m)
    ssa.ot_solve(prob, f, g, T, want_info=False)
    torch.cuda.synchronize()
    C = costs.cost_cosine(host64(X), host64(Y))
    f_ref, g_ref = oracle.sinkhorn(C, data["a"].astype(np.float64), data["b"].astype(np.float64),
                                   eps, T)
    df = np.abs(host64(f) - f_ref).max()
    dg = np.abs(host64(g) - g_ref).max()
    say(f"  max|df|={df:.2e} max|dg|={dg:.2e}")
    # bf16 points are normalised in fp32 and rounded to fp32 features: the
    # cost then differs from the oracle's only by fp32 rounding
    assert df <= POT_TOL["f32"] and dg <= POT_TOL["f32"]


@pytest.mark.parametrize("n,m,d,L,eps", [(333, 517, 16, 10, 0.1), (260, 300, 64, 7, 0.05),
                                         (150, 130, 200, 12, 0.1)])
def test_label_cost_solve_and_apply(n, m, d, L, eps):
    say(f"labels n={n} m={m} d={d} L={L} eps={eps}")
    data = workloads.make("c3_d16_f32", n=n, m=m, d=d)
    lab = workloads.label_inputs(n, m, L, seed=n + m + L)
    X, Y = _t(data["X"]), _t(data["Y"])
    a, b = _t(data["a"]), _t(data["b"])
    W = _t(lab["W"])
    Xa, sx = ssa.ot_prep_labels(X, _t(lab["lx"]), W, side=0)
    Ya, sy = ssa.ot_prep_labels(Y, _t(lab["ly"]), W, side=1)
    prob = ssa.problem(Xa, Ya, eps, a, b, x_sqn=sx, y_sqn=sy, affine=True)
    T = 30
    f, g = zeros(n), zeros(m)
    ssa.ot_solve(prob, f, g, T, want_info=False)
    torch.cuda.synchronize()
    a64, b64 = data["a"].astype(np.float64), data["b"].astype(np.float64)
    C = costs.cost_labels(data["X"], data["Y"], lab["lx"], lab["ly"], lab["W"])
    f_ref, g_ref = oracle.sinkhorn(C, a64, b64, eps, T)
    df = np.abs(host64(f) - f_ref).max()
    dg = np.abs(host64(g) - g_ref).max()
    say(f"  max|df|={df:.2e} max|dg|={dg:.2e}")
    assert df <= POT_TOL["f32"] and dg <= POT_TOL["f32"]
    f32, g32 = f_ref.astype(np.float32), g_ref.astype(np.float32)
    V = np.random.default_rng(L).standard_normal((m, 9)).astype(np.float32)
    pv = ssa.ot_apply_plan(prob, _t(f32), _t(g32), _t(V))
    torch.cuda.synchronize()
    P = oracle.plan(C, a64, b64, f32.astype(np.float64), g32.astype(np.float64), eps)
    ref = oracle.apply_plan(P, V.astype(np.float64))
    err = np.linalg.norm(host64(pv) - ref) / np.linalg.norm(ref)
    say(f"  P V rel err {err:.2e}")
    assert err <= PV_TOL


def test_label_cost_with_zero_w_equals_euclidean():
    """W = 0: the label features add nothing; the solve equals the plain squared-
    Euclidean solve of the same clouds up to the fp32 rounding of the two
    score paths."""
    n, m, d, L = 200, 170, 16, 5
    data = workloads.make("c3_d16_f32", n=n, m=m, d=d)
    lab = workloads.label_inputs(n, m, L, seed=4)
    X, Y = _t(data["X"]), _t(data["Y"])
    a, b = _t(data["a"]), _t(data["b"])
    Wz = torch.zeros((L, L), dtype=torch.float32, device=DEV)
    Xa, sx = ssa.ot_prep_labels(X, _t(lab["lx"]), Wz, side=0)
    Ya, sy = ssa.ot_prep_labels(Y, _t(lab["ly"]), Wz, side=1)
    f1, g1 = zeros(n), zeros(m)
    ssa.ot_solve(ssa.problem(Xa, Ya, 0.1, a, b, x_sqn=sx, y_sqn=sy, affine=True), f1, g1, 20,
                 want_info=False)
    f2, g2 = zeros(n), zeros(m)
    ssa.ot_solve(ssa.problem(X, Y, 0.1, a, b), f2, g2, 20, want_info=False)
    torch.cuda.synchronize()
    assert float((f1 - f2).abs().max()) <= 1e-4 and float((g1 - g2).abs().max()) <= 1e-4
