"""GPU parity at the full benchmark sizes, on sampled outputs.

Every workload runs at its full shape (up to n = 200000, d = 1024) through
the C ABI with the same entry points and the same automatic launch
configuration (column splits, tile shapes) that ``bench.py`` times. The dense
oracle cannot run those sizes, so the checks are teacher-forced on a seeded
sample of outputs, each computed by the oracle one row or one column at a
time, and every input of the oracle is seeded or the oracle's own:

* potentials f0 = ||x||^2 + u, g0 = ||y||^2 + v (norms from the oracle,
  offsets u, v ~ 0.1 N(0, 1) from ``workloads``), rounded to fp32, are given
  to both sides;
* f half-step: the GPU's ot_update_f from g0 (the pass shape and split count
  ot_solve uses) against the oracle's f-update of sampled rows i from g0;
* g half-step: ot_update_g from f0 against sampled columns;
* transport application of the coupling of (f0, g0): sampled rows of P V,
  r and the X-gradient, sampled columns of P^T U and c;
* the full solve (T iterations, launched as bench.py launches it) must end
  with finite potentials and small reported marginal errors.

Tolerances: 1e-4 (fp32 inputs) / 2e-2 (bf16 inputs) on potentials; relative
error 1e-4 on rows of P V, P^T U and the marginals for fp32 inputs. For bf16
inputs the P V gate is 1e-3, derived from the fp32 arithmetic of the score:
with identical potentials on both sides, ln P_ij carries the error of
(2/eps) x_i.y_j accumulated in fp32 over d/16 matrix steps, at most about
(2/eps) (d/16) 2^-24 max|x.y|. The 70000-point mixture workload (|x.y| up to
about 6, eps = 0.1, d = 512) bounds that by 2.3e-4 per entry.
"""

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_amd as ssa
import workloads
from gpu_util import DEV, host64, say, zeros

pytestmark = pytest.mark.gpu

POT_TOL = {"f32": 1e-4, "bf16": 2e-2}
PV_TOL = {"f32": 1e-4, "bf16": 1e-3}

FULL = ["c1", "c2", "c3_d16_f32", "c3_d128_f32", "c3_d512_f32", "c3_d1024_f32",
        "c3_d16_bf16", "c3_d128_bf16", "c3_d512_bf16", "c3_d1024_bf16", "c4", "c5"]

# Sample sizes keep the oracle's one-by-one evaluation to a few seconds even
# for the 200000 x 10000 x 1024 workload.
ROW_SAMPLES = {"c5": 24}
COL_SAMPLES = {"c5": 6, "c4": 16}


def _sample(count, k, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(count, size=min(k, count), replace=False)
    # always include both ends: the first row and the ragged last tile
    return np.unique(np.concatenate([idx, [0, count - 1]]))


def _to_dev(arr, dtype):
    t = torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    data = workloads.make(name)
    w = data["w"]
    T = w.iters
    say(f"full-size {name}: n={w.n} m={w.m} d={w.d} {w.dtype} eps={w.eps} T={T}")
    X = _to_dev(data["X"], w.dtype)
    Y = _to_dev(data["Y"], w.dtype)
    a = torch.from_numpy(data["a"]).to(DEV)
    b = torch.from_numpy(data["b"]).to(DEV)
    prob = ssa.problem(X, Y, w.eps, a, b)
    Xh, Yh = host64(X), host64(Y)
    ah, bh = data["a"].astype(np.float64), data["b"].astype(np.float64)
    u, v = workloads.potential_offsets(w.n, w.m, seed=w.config * 100 + w.variant)
    f0 = (oracle.sqnorms(Xh) + u).astype(np.float32)
    g0 = (oracle.sqnorms(Yh) + v).astype(np.float32)
    f0h, g0h = f0.astype(np.float64), g0.astype(np.float64)
    tol = POT_TOL[w.dtype]
    rows = _sample(w.n, ROW_SAMPLES.get(name, 64), 1)
    cols = _sample(w.m, COL_SAMPLES.get(name, 32), 2)

    # Teacher-forced half-steps.
    f = torch.from_numpy(f0).to(DEV)
    g = torch.from_numpy(g0).to(DEV)
    f1, g1 = f.clone(), g.clone()
    ssa.ot_update_f(prob, g, f1)
    ssa.ot_update_g(prob, f, g1)
    torch.cuda.synchronize()
    df = np.abs(host64(f1)[rows] - oracle.update_f_rows(Xh[rows], Yh, g0h, bh, w.eps)).max()
    dg = np.abs(host64(g1)[cols] - oracle.update_g_cols(Xh, Yh[cols], f0h, ah, w.eps)).max()
    say(f"  half-steps: sampled max|df|={df:.3e} ({len(rows)} rows)  max|dg|={dg:.3e} ({len(cols)} cols)")
    assert df <= tol and dg <= tol

    # Transport application of the coupling of (f0, g0).
    Prow = oracle.plan_rows(Xh[rows], Yh, ah[rows], bh, f0h[rows], g0h, w.eps)
    if w.grad:
        grad = ssa.ot_apply_plan(prob, f, g, flags=ssa.OT_GRAD)
        torch.cuda.synchronize()
        g_ref_rows = 2.0 * (Prow.sum(axis=1)[:, None] * Xh[rows] - Prow @ Yh)
        err = np.linalg.norm(host64(grad)[rows] - g_ref_rows) / np.linalg.norm(g_ref_rows)
        say(f"  grad rows rel err {err:.3e}")
        assert err <= 10 * PV_TOL[w.dtype]
    if w.v_cols:
        V = _to_dev(data["V"], w.dtype)
        r = torch.empty(w.n, dtype=torch.float32, device=DEV)
        pv = ssa.ot_apply_plan(prob, f, g, V, marg=r)
        torch.cuda.synchronize()
        ref = Prow @ host64(V)
        err = np.linalg.norm(host64(pv)[rows] - ref) / np.linalg.norm(ref)
        rerr = np.abs(host64(r)[rows] - Prow.sum(axis=1)).max() / Prow.sum(axis=1).max()
        say(f"  P V rows rel err {err:.3e}, r rel err {rerr:.3e}")
        assert err <= PV_TOL[w.dtype] and rerr <= PV_TOL[w.dtype]
    if w.u_cols:
        U = _to_dev(data["U"], w.dtype)
        c = torch.empty(w.m, dtype=torch.float32, device=DEV)
        ptu = ssa.ot_apply_plan(prob, f, g, U, flags=ssa.OT_TRANSPOSE, marg=c)
        torch.cuda.synchronize()
        Pcol = oracle.plan_cols(Xh, Yh[cols], ah, bh[cols], f0h, g0h[cols], w.eps)
        ref = Pcol.T @ host64(U)
        err = np.linalg.norm(host64(ptu)[cols] - ref) / np.linalg.norm(ref)
        cerr = np.abs(host64(c)[cols] - Pcol.sum(axis=0)).max() / Pcol.sum(axis=0).max()
        say(f"  P^T U cols rel err {err:.3e}, c rel err {cerr:.3e}")
        assert err <= PV_TOL[w.dtype] and cerr <= PV_TOL[w.dtype]

    # The full solve as bench.py runs it: T iterations from zero potentials.
    fs, gs = zeros(w.n), zeros(w.m)
    info = ssa.ot_solve(prob, fs, gs, T, timing=True)
    torch.cuda.synchronize()
    say(f"  solve: splits f/g = {info['splits_f']}/{info['splits_g']}, marg err row "
        f"{info['marg_err_row']:.3e} col {info['marg_err_col']:.3e}")
    assert not info["nonfinite"] and info["iters_done"] == T
    # the last half-step fits the columns; the rows are within the iteration's progress
    assert info["marg_err_col"] <= 1e-3 and info["marg_err_row"] <= 1e-2
