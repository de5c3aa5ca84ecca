"""GPU parity of the second-order entry points against the fp64 oracle.

* ``ot_apply_hadamard``: (P . A Y^T) V (Algorithm 5) against the dense oracle
  product on the same potentials.
* ``ot_hvp``: T A against ``oracle.hvp.hvp_schur_cg`` with the same damping
  tau, iteration cap K and tolerance eta, on the page's parity shape
  (App. H.2.3: n = m = 512, d = 4, X, Y ~ N(0, I), random simplex weights,
  eps in {0.1, 0.25, 0.5}) and on ragged shapes spanning several tiles.

Inputs are seeded (``workloads`` draws the clouds; the potentials are the
oracle's own Sinkhorn iterates, rounded to fp32 and given to both sides).

Tolerances (relative Frobenius error of G):
* converged solve (eta = 1e-6): the same solve carried out in fp32 arithmetic
  on the CPU differs from fp64 by at most 6e-6 on the page's shape, so the
  bar is 1e-4 (PV_TOL, the fp32 transport-product bar);
* K = 50 fixed iterations, tau = 1e-5 (the page's benchmark setting, App.
  H.2): the solve has not converged, and the fp32 recurrence drifts from the
  fp64 one by up to 2.6e-4 on the page's shape; the bar is 2e-3.
"""

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_amd as ssa
import workloads
from oracle import hvp as H
from gpu_util import DEV, host64, say

pytestmark = pytest.mark.gpu

PV_TOL = 1e-4
FIXED_K_TOL = 2e-3


def _rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def _setup(n, m, d, eps, seed, iters=200):
    """Seeded clouds (page's HVP parity recipe), oracle potentials rounded to fp32."""
    data = workloads.hvp_parity_inputs(n, m, d, seed)
    X32, Y32, A32 = data["X"], data["Y"], data["A"]
    a32, b32 = data["a"], data["b"]
    X, Y, a, b = (v.astype(np.float64) for v in (X32, Y32, a32, b32))
    f, g = oracle.sinkhorn(oracle.cost_matrix(X, Y), a, b, eps, iters)
    f32, g32 = f.astype(np.float32), g.astype(np.float32)
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    prob = ssa.problem(t(X32), t(Y32), eps, t(a32), t(b32))
    host = dict(X=X, Y=Y, a=a, b=b, A=A32.astype(np.float64), f=f32.astype(np.float64),
                g=g32.astype(np.float64))
    return prob, t(f32), t(g32), t(A32), host


HAD_CASES = [
    # n, m, d, cols, eps: resident layouts (d <= 128, one chunk of up to 8
    # k-blocks) and the chunked layout (d > 128), ragged tails everywhere
    (100, 77, 4, 5, 0.25),
    (333, 517, 16, 33, 0.1),
    (150, 210, 70, 64, 0.5),
    (97, 130, 200, 3, 0.5),
]


@pytest.mark.parametrize("n,m,d,cols,eps", HAD_CASES)
def test_apply_hadamard(n, m, d, cols, eps):
    say(f"hadamard n={n} m={m} d={d} cols={cols} eps={eps}")
    prob, f, g, A, h = _setup(n, m, d, eps, seed=n + m + d, iters=30)
    V32 = np.random.default_rng(d).standard_normal((m, cols)).astype(np.float32)
    out = ssa.ot_apply_hadamard(prob, f, g, A, torch.from_numpy(V32).to(DEV))
    torch.cuda.synchronize()
    P = oracle.plan(oracle.cost_matrix(h["X"], h["Y"]), h["a"], h["b"], h["f"], h["g"], eps)
    W = h["A"] @ h["Y"].T
    V = V32.astype(np.float64)
    ref = (P * W) @ V
    # the weights have mixed signs: measure against the magnitude sum
    scale = np.linalg.norm((P * np.abs(W)) @ np.abs(V))
    err = np.linalg.norm(host64(out) - ref) / scale
    say(f"  rel err {err:.2e}")
    assert err <= PV_TOL


HVP_CASES = [
    # n, m, d, eps: the page's parity shape, then ragged shapes over several tiles
    (512, 512, 4, 0.1),
    (512, 512, 4, 0.25),
    (512, 512, 4, 0.5),
    (333, 517, 16, 0.25),
    (150, 210, 70, 0.5),
    (97, 130, 200, 0.5),
]


@pytest.mark.parametrize("n,m,d,eps", HVP_CASES)
def test_hvp_converged(n, m, d, eps):
    say(f"hvp converged n={n} m={m} d={d} eps={eps}")
    prob, f, g, A, h = _setup(n, m, d, eps, seed=7 * n + d)
    G, info = ssa.ot_hvp(prob, f, g, A, tau=1e-5, max_iters=500, tol=1e-6)
    torch.cuda.synchronize()
    ref, k, rel = H.hvp_schur_cg(h["X"], h["Y"], h["a"], h["b"], h["f"], h["g"], eps, h["A"],
                                 tau=1e-5, iters=500, tol=1e-6)
    err = _rel(host64(G), ref)
    say(f"  rel err {err:.2e}; cg iters gpu {info['cg_iters']} oracle {k}; "
        f"residual {info['cg_rel_residual']:.2e}")
    assert not info["breakdown"]
    assert info["cg_rel_residual"] <= 1e-6
    assert info["cg_iters"] <= 500
    assert err <= PV_TOL


@pytest.mark.parametrize("eps", [0.1, 0.5])
def test_hvp_fixed_iterations(eps):
    """The page's benchmark setting: K = 50, tau = 1e-5, no early stop."""
    say(f"hvp K=50 eps={eps}")
    prob, f, g, A, h = _setup(512, 512, 4, eps, seed=11)
    G, info = ssa.ot_hvp(prob, f, g, A, tau=1e-5, max_iters=50, tol=0.0)
    torch.cuda.synchronize()
    ref, k, _ = H.hvp_schur_cg(h["X"], h["Y"], h["a"], h["b"], h["f"], h["g"], eps, h["A"],
                               tau=1e-5, iters=50, tol=0.0)
    err = _rel(host64(G), ref)
    say(f"  rel err {err:.2e}")
    assert info["cg_iters"] == 50 == k
    assert err <= FIXED_K_TOL


def test_hvp_without_solve_is_explicit_plus_backsubstitution():
    """K = 0: w2 = 0 and w1 = R1 / r; compared with the oracle taking the same path."""
    prob, f, g, A, h = _setup(200, 150, 8, 0.3, seed=3)
    G, info = ssa.ot_hvp(prob, f, g, A, tau=1e-5, max_iters=0)
    torch.cuda.synchronize()
    ref, k, _ = H.hvp_schur_cg(h["X"], h["Y"], h["a"], h["b"], h["f"], h["g"], 0.3, h["A"],
                               tau=1e-5, iters=0)
    assert info["cg_iters"] == 0 == k
    assert _rel(host64(G), ref) <= PV_TOL


def test_hvp_single_target_closed_form():
    """m = 1: T A = 2 a * A whatever the solve does (S = 0, and the
    back-substitution makes w1_i + w2 = R1_i / r_i)."""
    rng = np.random.default_rng(5)
    n, d, eps = 300, 6, 0.2
    X32 = rng.standard_normal((n, d)).astype(np.float32)
    Y32 = rng.standard_normal((1, d)).astype(np.float32)
    a32 = rng.dirichlet(np.ones(n)).astype(np.float32)
    b32 = np.ones(1, dtype=np.float32)
    A32 = rng.standard_normal((n, d)).astype(np.float32)
    t = lambda v: torch.from_numpy(v).to(DEV)
    X, Y, a, b = (v.astype(np.float64) for v in (X32, Y32, a32, b32))
    f, g = oracle.sinkhorn(oracle.cost_matrix(X, Y), a, b, eps, 5)
    prob = ssa.problem(t(X32), t(Y32), eps, t(a32), t(b32))
    G, _ = ssa.ot_hvp(prob, t(f.astype(np.float32)), t(g.astype(np.float32)), t(A32),
                      tau=1e-5, max_iters=20, tol=1e-6)
    torch.cuda.synchronize()
    # r = a up to the fp32 potentials: compare with 2 r * A of the same potentials
    r, _ = oracle.marginals(oracle.plan(oracle.cost_matrix(X, Y), a, b,
                                        f.astype(np.float32).astype(np.float64),
                                        g.astype(np.float32).astype(np.float64), eps))
    assert _rel(host64(G), 2.0 * r[:, None] * A32.astype(np.float64)) <= PV_TOL


def test_hvp_zero_direction_is_zero_and_repeatable():
    prob, f, g, A, h = _setup(130, 90, 5, 0.4, seed=9)
    Z = torch.zeros_like(A)
    G0, info = ssa.ot_hvp(prob, f, g, Z, max_iters=10)
    torch.cuda.synchronize()
    assert info["cg_iters"] == 0 and not torch.any(G0)
    G1, _ = ssa.ot_hvp(prob, f, g, A, max_iters=30)
    G2, _ = ssa.ot_hvp(prob, f, g, A, max_iters=30)
    torch.cuda.synchronize()
    assert torch.equal(G1, G2)


def test_hvp_is_symmetric():
    """<B, T A> = <A, T B> for the converged solve (the Hessian is symmetric)."""
    prob, f, g, A, h = _setup(256, 300, 4, 0.25, seed=21)
    B = torch.from_numpy(np.random.default_rng(22).standard_normal((256, 4)).astype(np.float32)).to(DEV)
    GA, _ = ssa.ot_hvp(prob, f, g, A, tau=1e-6, max_iters=1000, tol=1e-7)
    GB, _ = ssa.ot_hvp(prob, f, g, B, tau=1e-6, max_iters=1000, tol=1e-7)
    torch.cuda.synchronize()
    lhs = float(torch.sum(B.double() * GA.double()))
    rhs = float(torch.sum(A.double() * GB.double()))
    scale = float(torch.linalg.norm(B.double()) * torch.linalg.norm(GA.double()))
    assert abs(lhs - rhs) <= 1e-4 * scale


@pytest.mark.parametrize("mode", ["native", "split_bf16"])
@pytest.mark.parametrize("n,m,d,eps", [(200, 150, 8, 0.3), (130, 90, 70, 0.5)])
def test_hvp_other_fp32_operand_modes(n, m, d, eps, mode):
    """OT_NATIVE_F32 / OT_SPLIT_BF16: the conjugate-gradient passes form scores
    with the fp32 matrix instruction or from three bf16 parts (register-
    pipelined kernel for d = 8, LDS-shared for d = 70)."""
    say(f"hvp {mode} n={n} m={m} d={d} eps={eps}")
    data = workloads.hvp_parity_inputs(n, m, d, seed=n + d)
    X, Y, a, b = (data[k].astype(np.float64) for k in ("X", "Y", "a", "b"))
    f, g = oracle.sinkhorn(oracle.cost_matrix(X, Y), a, b, eps, 200)
    f32, g32 = f.astype(np.float32), g.astype(np.float32)
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    prob = ssa.problem(t(data["X"]), t(data["Y"]), eps, t(data["a"]), t(data["b"]),
                       native_f32=mode == "native", split_bf16=mode == "split_bf16")
    G, info = ssa.ot_hvp(prob, t(f32), t(g32), t(data["A"]), tau=1e-5, max_iters=500, tol=1e-6)
    torch.cuda.synchronize()
    ref, _, _ = H.hvp_schur_cg(X, Y, a, b, f32.astype(np.float64), g32.astype(np.float64), eps,
                               data["A"].astype(np.float64), tau=1e-5, iters=500, tol=1e-6)
    err = _rel(host64(G), ref)
    say(f"  rel err {err:.2e}, cg iters {info['cg_iters']}")
    assert err <= PV_TOL


def test_hvp_range_exceeded_reported():
    """Clouds too large for the two-part fp16 scores: ot_hvp reports
    OT_ERR_UNSUPPORTED (with or without info) instead of returning a NaN
    product, and leaves its output unwritten."""
    data = workloads.hvp_parity_inputs(60, 50, 6, seed=3)
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    prob = ssa.problem(t(data["X"] * 1e5), t(data["Y"] * 1e5), 1.0, t(data["a"]), t(data["b"]))
    f, g = torch.zeros(60, device=DEV), torch.zeros(50, device=DEV)
    for want_info in (True, False):
        out = torch.full((60, 6), 7.0, device=DEV)
        with pytest.raises(ssa.OtError) as ei:
            ssa.ot_hvp(prob, f, g, t(data["A"]), tau=1e-5, max_iters=3, out=out, want_info=want_info)
        torch.cuda.synchronize()
        assert ei.value.code == ssa.OT_ERR_UNSUPPORTED
        assert bool((out == 7.0).all())


def test_hvp_tiny_single_partial_tile():
    """n, m below one 32-row tile: every tile is ragged."""
    prob, f, g, A, h = _setup(5, 7, 3, 0.4, seed=13, iters=100)
    G, info = ssa.ot_hvp(prob, f, g, A, tau=1e-6, max_iters=50, tol=1e-7)
    torch.cuda.synchronize()
    ref, _, _ = H.hvp_schur_cg(h["X"], h["Y"], h["a"], h["b"], h["f"], h["g"], 0.4, h["A"],
                               tau=1e-6, iters=50, tol=1e-7)
    assert _rel(host64(G), ref) <= PV_TOL
