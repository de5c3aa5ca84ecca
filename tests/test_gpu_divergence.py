"""GPU parity of eps-scaling and the debiased Sinkhorn divergence against the
fp64 oracle (``oracle.divergence``).

Tolerances: potentials 1e-4 for fp32 points (2e-2 for bf16), as for the
plain solve. Each dual value <a, f> + <b, g> then differs by at most the
potential bar (weights sum to one on each side): 2e-4; S combines one full
and two half dual values, so its bar is 4e-4 absolute.
"""

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_amd as ssa
import workloads
from oracle import divergence as D
from gpu_util import host64, make_problem, oracle_inputs, say, zeros

pytestmark = pytest.mark.gpu

POT_TOL = {"f32": 1e-4, "bf16": 2e-2}

SCALING_CASES = [
    # workload, n, m, d, iters, eps_start, decay, schedule
    ("c2", 700, 555, None, 40, 1.0, 0.5, "alternating"),
    ("c3_d128_f32", 400, 330, None, 30, 2.0, 0.7, "alternating"),
    ("c3_d512_bf16", 300, 260, None, 30, 1.0, 0.5, "alternating"),
    ("c5", 1000, 120, 256, 60, 1.0, 0.8, "alternating"),
    ("c2", 600, 500, None, 40, 1.0, 0.5, "symmetric"),
    ("c1", None, None, None, 3, 1.0, 0.5, "alternating"),     # all iterations annealed
]


@pytest.mark.parametrize("case", SCALING_CASES, ids=lambda c: f"{c[0]}-{c[7]}-{c[4]}")
def test_eps_scaling_trajectory(case):
    name, n, m, d, T, e0, q, sched = case
    data = workloads.make(name, n=n, m=m, d=d)
    w = data["w"]
    say(f"eps-scaling {name} n={w.n} m={w.m} d={w.d} {w.dtype} eps={w.eps} T={T} from {e0} x{q} {sched}")
    prob = make_problem(data)
    X, Y, a, b = oracle_inputs(prob)
    f, g = zeros(w.n), zeros(w.m)
    info = ssa.ot_solve(prob, f, g, T, schedule=sched, eps_start=e0, eps_decay=q)
    torch.cuda.synchronize()
    C = oracle.cost_matrix(X, Y)
    f_ref, g_ref = D.sinkhorn_eps_scaling(C, a, b, w.eps, T, e0, q, schedule=sched)
    df = np.abs(host64(f) - f_ref).max()
    dg = np.abs(host64(g) - g_ref).max()
    say(f"  max|df|={df:.2e} max|dg|={dg:.2e}")
    assert info["iters_done"] == T and not info["nonfinite"]
    assert df <= POT_TOL[w.dtype] and dg <= POT_TOL[w.dtype]
    # The reported marginal errors are those of the returned potentials at the
    # problem's eps, also when every iteration ran at a larger eps_k (then the
    # columns are not fit either). The returned potentials differ from the
    # oracle's by at most df, dg, so every coupling entry by a factor within
    # exp(+-(df + dg)/eps): the L1 errors by at most expm1((df + dg)/eps) sum(P).
    P = oracle.plan(C, a, b, f_ref, g_ref, w.eps)
    er, ec = oracle.marginal_errors(P, a, b)
    bound = np.expm1((df + dg) / w.eps) * P.sum() * 1.01 + 2e-6
    say(f"  marg err row {info['marg_err_row']:.3e} (oracle {er:.3e}), "
        f"col {info['marg_err_col']:.3e} (oracle {ec:.3e}), bound {bound:.1e}")
    assert abs(info["marg_err_row"] - er) <= bound + 1e-2 * er
    assert abs(info["marg_err_col"] - ec) <= bound + 1e-2 * ec


def test_eps_scaling_then_plain_graph_replay_is_repeatable():
    """The annealed iterations and the graph-replayed ones compose the same way
    in two calls, and the graph cached for the target eps is not disturbed."""
    data = workloads.make("c2", n=900, m=800)
    prob = make_problem(data)
    outs = []
    for _ in range(2):
        f, g = zeros(900), zeros(800)
        ssa.ot_solve(prob, f, g, 40, eps_start=1.0, eps_decay=0.5, want_info=False)
        outs.append((f.clone(), g.clone()))
    f, g = zeros(900), zeros(800)
    ssa.ot_solve(prob, f, g, 40, want_info=False)
    f2, g2 = zeros(900), zeros(800)
    ssa.ot_solve(prob, f2, g2, 40, want_info=False, use_graph=False)
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(f, f2) and torch.equal(g, g2)


DIV_CASES = [
    # workload, n, m, d, iters, eps_start, schedule
    ("c1", 400, 300, None, 60, 0.0, "alternating"),
    ("c2", 500, 450, None, 50, 1.0, "alternating"),
    ("c3_d128_bf16", 300, 350, None, 40, 0.0, "alternating"),
    ("c3_d16_f32", 380, 290, None, 50, 0.0, "symmetric"),
]


@pytest.mark.parametrize("case", DIV_CASES, ids=lambda c: f"{c[0]}-{c[6]}")
def test_sinkhorn_divergence(case):
    name, n, m, d, T, e0, sched = case
    data = workloads.make(name, n=n, m=m, d=d)
    w = data["w"]
    say(f"divergence {name} n={w.n} m={w.m} d={w.d} {w.dtype} T={T} eps_start={e0} {sched}")
    prob = make_problem(data)
    X, Y, a, b = oracle_inputs(prob)
    vals, f, g, fxx, gyy = ssa.ot_sinkhorn_divergence(prob, T, schedule=sched, eps_start=e0,
                                                       eps_decay=0.5)
    ref = D.sinkhorn_divergence(X, Y, a, b, w.eps, T, eps_start=e0, decay=0.5, schedule=sched)
    tol = POT_TOL[w.dtype]
    for got, want, name_ in ((f, ref[4], "f"), (g, ref[5], "g"), (fxx, ref[6], "f_xx"),
                             (gyy, ref[7], "g_yy")):
        err = np.abs(host64(got) - want).max()
        say(f"  max|d{name_}|={err:.2e}")
        assert err <= tol
    say(f"  S gpu {vals[0]:.6e} oracle {ref[0]:.6e}; OT values {vals[1:]} vs {ref[1:4]}")
    assert abs(vals[0] - ref[0]) <= 4 * tol
    for k in (1, 2, 3):
        assert abs(vals[k] - ref[k]) <= 2 * tol


def test_divergence_of_identical_clouds_is_zero():
    data = workloads.make("c3_d16_f32", n=300, m=300)
    data["Y"] = data["X"].copy()
    data["b"] = data["a"].copy()
    prob = make_problem(data)
    vals, *_ = ssa.ot_sinkhorn_divergence(prob, 30)
    # the three solves are bit-identical runs of the same problem
    assert vals[0] == 0.0
