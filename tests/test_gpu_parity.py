"""GPU parity of the HIP path against the fp64 oracle, element by element.

All calls go through the C ABI (via the ctypes binding). Sizes are chosen so
that the dense oracle finishes in seconds while the GPU side spans several
32-row tiles, several column splits and a ragged tail. Tolerances are the
ones the project is held to: max |df|, |dg| <= 1e-4 for fp32 inputs and
<= 2e-2 for bf16 inputs; relative Frobenius error of P V <= 1e-4 for fp32
with identical potentials fed to both sides (bf16 inputs use the same gate:
the oracle receives the exact bf16 values, so only fp32 rounding separates
the two sides).
"""

import numpy as np
import pytest
import torch

import oracle
import streaming_sinkhorn_amd as ssa
import workloads
from gpu_util import DEV, F32_MODES, dev, host64, make_problem, oracle_inputs, say, zeros

pytestmark = pytest.mark.gpu

POT_TOL = {"f32": 1e-4, "bf16": 2e-2}
PV_TOL = 1e-4


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --- building blocks -------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,d", [(1, 1), (37, 3), (100, 64), (333, 1000)])
def test_sqnorms(dtype, rows, d):
    say(f"sqnorms dtype={dtype} rows={rows} d={d}")
    data = workloads.make("c3_d16_f32", n=rows, m=1, d=d)
    X = torch.from_numpy(data["X"]).to(DEV)
    if dtype == "bf16":
        X = X.to(torch.bfloat16)
    out = ssa.ot_sqnorms(X)
    torch.cuda.synchronize()
    ref = oracle.sqnorms(host64(X))
    np.testing.assert_allclose(host64(out), ref, rtol=2e-6, atol=1e-6)


# --- single half-steps (teacher-forced: identical inputs on both sides) -----------

def with_modes(cases):
    """Each case once per fp32 operand mode for fp32 points; bf16 points have
    one operand mode (the modes only choose how fp32 values are multiplied)."""
    out = []
    for case in cases:
        modes = F32_MODES if case[3] == "f32" else F32_MODES[:1]
        out += [(*case, mode) for mode in modes]
    return out


HALF_CASES = [
    # (n, m, d, dtype, eps)
    (333, 517, 16, "f32", 0.1),
    (517, 333, 64, "f32", 0.1),
    (70, 1500, 1, "f32", 0.1),
    (129, 95, 3, "f32", 0.05),
    (260, 300, 17, "f32", 0.1),
    (300, 260, 100, "f32", 0.1),
    (200, 190, 128, "f32", 0.1),
    (150, 210, 200, "f32", 0.1),
    (120, 140, 512, "f32", 0.1),
    (97, 64, 1024, "f32", 0.01),
    (333, 517, 16, "bf16", 0.1),
    (300, 260, 64, "bf16", 0.1),
    (200, 190, 128, "bf16", 0.1),
    (150, 210, 256, "bf16", 0.1),
    (120, 140, 512, "bf16", 0.1),
    (97, 64, 1024, "bf16", 0.01),
    # eps = 0.01 with few column tiles: scores far below zero in log2 units,
    # where a tile folded before the row's stabiliser was set must take the
    # exact path (its rescale factor would overflow)
    (300, 40, 64, "f32", 0.01),
    (260, 70, 17, "bf16", 0.01),
    (150, 90, 300, "f32", 0.01),
    # passes with the lazily raised stabiliser (at most three score MFMAs per
    # tile: fp16 split d <= 16, bf16 d <= 48), also at eps = 0.01
    (300, 40, 16, "f32", 0.01),
    (210, 170, 40, "bf16", 0.05),
    (180, 45, 48, "bf16", 0.01),
]


# fp32 cases run in every fp32 operand mode: resident (d <= 128, LDS-shared
# columns from d = 64) and the tiled wide pass (d > 128)
@pytest.mark.parametrize("n,m,d,dtype,eps,mode", with_modes(HALF_CASES))
def test_half_steps_teacher_forced(n, m, d, dtype, eps, mode):
    say(f"half-steps n={n} m={m} d={d} dtype={dtype} eps={eps} mode={mode}")
    base = "c3_d16_bf16" if dtype == "bf16" else "c3_d16_f32"
    data = workloads.make(base, n=n, m=m, d=d)
    prob = make_problem(data, eps=eps, mode=mode)
    X, Y, a, b = oracle_inputs(prob)
    C = oracle.cost_matrix(X, Y)
    rng = np.random.default_rng(n * 7 + m)
    g0 = (rng.standard_normal(m) * 0.3).astype(np.float32)
    f0 = (rng.standard_normal(n) * 0.3).astype(np.float32)
    g = torch.from_numpy(g0).to(DEV)
    f = torch.from_numpy(f0).to(DEV)
    err = torch.zeros(1, dtype=torch.float32, device=DEV)
    ssa.ot_update_f(prob, g, f, err=err)
    torch.cuda.synchronize()
    f_ref = oracle.update_f(C, g0.astype(np.float64), b, eps)
    tol = POT_TOL[dtype]
    df = np.abs(host64(f) - f_ref).max()
    assert df <= tol, f"max|df| = {df}"
    # err = ||P(f0, g0) 1 - a||_1
    r, _ = oracle.marginals(oracle.plan(C, a, b, f0.astype(np.float64), g0.astype(np.float64), eps))
    e_ref = np.abs(r - a).sum()
    assert abs(float(err.item()) - e_ref) <= 1e-3 * max(e_ref, 1.0)
    # g half-step from the oracle's f (rounded to fp32, given to both sides)
    f1 = f_ref.astype(np.float32)
    g2 = torch.from_numpy(g0).to(DEV)
    ssa.ot_update_g(prob, torch.from_numpy(f1).to(DEV), g2, err=err)
    torch.cuda.synchronize()
    g_ref = oracle.update_g(C, f1.astype(np.float64), a, eps)
    dg = np.abs(host64(g2) - g_ref).max()
    assert dg <= tol, f"max|dg| = {dg}"
    # err = ||P(f1, g0)^T 1 - b||_1
    _, c = oracle.marginals(oracle.plan(C, a, b, f1.astype(np.float64), g0.astype(np.float64), eps))
    e_ref = np.abs(c - b).sum()
    assert abs(float(err.item()) - e_ref) <= 1e-3 * max(e_ref, 1.0)


# --- full trajectories ----------------------------------------------------------------

TRAJ_CASES = [
    # workload, n, m, d override (None = workload's), iters override
    ("c1", None, None, None, None),
    ("c2", 700, 555, None, None),
    ("c3_d16_f32", 500, 650, None, None),
    ("c3_d128_f32", 500, 650, None, None),
    ("c3_d512_f32", 300, 420, None, None),
    ("c3_d1024_f32", 300, 250, None, None),
    ("c3_d16_bf16", 500, 650, None, None),
    ("c3_d128_bf16", 500, 650, None, None),
    ("c3_d512_bf16", 300, 420, None, None),
    ("c3_d1024_bf16", 300, 250, None, None),
    ("c4", 800, 700, None, 200),
    ("c5", 1000, 120, None, 300),
    # the eps = 0.01 workload at d = 16: passes with the lazily raised
    # stabiliser over 300 iterations
    ("c5", 600, 300, 16, 300),
]


TRAJ_CASES += [
    # the same fp32 workloads formed with the fp32 matrix instruction and
    # with the three-part bf16 split
    (*c, mode) for mode in ("native", "split_bf16") for c in [
        ("c1", None, None, None, None),
        ("c2", 700, 555, None, None),
        ("c3_d16_f32", 500, 650, None, None),
        ("c3_d128_f32", 500, 650, None, None),
        ("c3_d512_f32", 300, 420, None, None),
    ]
]


@pytest.mark.parametrize("case", TRAJ_CASES, ids=lambda c: "-".join(str(v) for v in c if v is not None))
def test_solve_trajectory(case):
    name, n, m, d, iters = case[:5]
    mode = case[5] if len(case) > 5 else "half2"
    data = workloads.make(name, n=n, m=m, d=d)
    w = data["w"]
    T = w.iters if iters is None else iters
    say(f"trajectory {name} n={w.n} m={w.m} d={w.d} dtype={w.dtype} eps={w.eps} T={T} mode={mode}")
    prob = make_problem(data, mode=mode)
    X, Y, a, b = oracle_inputs(prob)
    f = zeros(w.n)
    g = zeros(w.m)
    info = ssa.ot_solve(prob, f, g, T)
    torch.cuda.synchronize()
    C = oracle.cost_matrix(X, Y)
    f_ref, g_ref = oracle.sinkhorn(C, a, b, w.eps, T)
    tol = POT_TOL[w.dtype]
    df = np.abs(host64(f) - f_ref).max()
    dg = np.abs(host64(g) - g_ref).max()
    say(f"  max|df|={df:.3e} max|dg|={dg:.3e} info={info}")
    assert df <= tol and dg <= tol
    assert info["iters_done"] == T and not info["nonfinite"]
    _check_reported_marginals(info, C, a, b, f_ref, g_ref, w.eps, df, dg)


def _check_reported_marginals(info, C, a, b, f_ref, g_ref, eps, df, dg):
    """The reported exact marginal errors are those of the returned potentials.
    They are compared with the oracle's errors of its own potentials: the
    returned ones differ by at most df, dg, so each entry of the coupling
    differs by a factor within exp(+-(df + dg)/eps) and the L1 errors by at
    most expm1((df + dg)/eps) * sum(P)."""
    P = oracle.plan(C, a, b, f_ref, g_ref, eps)
    er, ec = oracle.marginal_errors(P, a, b)
    bound = np.expm1((df + dg) / eps) * P.sum() * 1.01 + 2e-6
    assert abs(info["marg_err_row"] - er) <= bound + 1e-2 * er
    assert abs(info["marg_err_col"] - ec) <= bound + 1e-2 * ec


# --- symmetric schedule ---------------------------------------------------------------

SYM_CASES = [
    # workload, n, m, d override, iters
    ("c1", None, None, None, 30),
    ("c2", 700, 555, None, 60),
    ("c3_d16_bf16", 500, 650, None, 40),
    ("c3_d128_f32", 400, 330, None, 40),
    ("c3_d512_f32", 300, 420, None, 30),
    ("c3_d1024_bf16", 260, 200, None, 30),
    ("c5", 1000, 120, None, 60),
]


@pytest.mark.parametrize("case", SYM_CASES, ids=lambda c: c[0])
def test_solve_symmetric_trajectory(case):
    """Symmetric (averaged) schedule against the oracle's symmetric iteration."""
    name, n, m, d, T = case
    data = workloads.make(name, n=n, m=m, d=d)
    w = data["w"]
    say(f"symmetric {name} n={w.n} m={w.m} d={w.d} dtype={w.dtype} eps={w.eps} T={T}")
    prob = make_problem(data)
    X, Y, a, b = oracle_inputs(prob)
    f, g = zeros(w.n), zeros(w.m)
    info = ssa.ot_solve(prob, f, g, T, schedule="symmetric")
    torch.cuda.synchronize()
    C = oracle.cost_matrix(X, Y)
    f_ref, g_ref = oracle.sinkhorn_symmetric(C, a, b, w.eps, T)
    df = np.abs(host64(f) - f_ref).max()
    dg = np.abs(host64(g) - g_ref).max()
    say(f"  max|df|={df:.3e} max|dg|={dg:.3e}")
    tol = POT_TOL[w.dtype]
    assert df <= tol and dg <= tol
    _check_reported_marginals(info, C, a, b, f_ref, g_ref, w.eps, df, dg)


def test_symmetric_graph_eager_and_resume_bitwise():
    data = workloads.make("c2", n=1100, m=900)
    prob = make_problem(data)
    outs = []
    for use_graph in (True, False):
        f, g = zeros(1100), zeros(900)
        ssa.ot_solve(prob, f, g, 21, use_graph=use_graph, want_info=False, schedule="symmetric")
        outs.append((f.clone(), g.clone()))
    f, g = zeros(1100), zeros(900)
    ssa.ot_solve(prob, f, g, 9, want_info=False, schedule="symmetric")
    ssa.ot_solve(prob, f, g, 12, init_given=True, want_info=False, schedule="symmetric")
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(f, outs[0][0]) and torch.equal(g, outs[0][1])


# --- transport application ------------------------------------------------------------

APPLY_CASES = [
    # n, m, d, dtype, eps, cols
    (333, 517, 16, "f32", 0.1, 64),
    (517, 333, 64, "f32", 0.1, 64),
    (300, 260, 128, "f32", 0.1, 128),
    (200, 150, 1024, "f32", 0.01, 128),
    (260, 300, 64, "bf16", 0.1, 64),
    (150, 170, 512, "bf16", 0.1, 33),
    (90, 75, 17, "f32", 0.05, 1),
    (64, 1, 8, "f32", 0.1, 5),
    (170, 190, 300, "f32", 0.1, 20),
]


@pytest.mark.parametrize("n,m,d,dtype,eps,cols,mode", with_modes(APPLY_CASES))
def test_apply_plan(n, m, d, dtype, eps, cols, mode):
    """Default operands: scores and value product from fp16 parts (bf16 scores
    for bf16 points); OT_NATIVE_F32 / OT_SPLIT_BF16: the fp32 kernel."""
    say(f"apply n={n} m={m} d={d} dtype={dtype} eps={eps} cols={cols} mode={mode}")
    base = "c3_d16_bf16" if dtype == "bf16" else "c3_d16_f32"
    data = workloads.make(base, n=n, m=m, d=d)
    prob = make_problem(data, eps=eps, mode=mode)
    X, Y, a, b = oracle_inputs(prob)
    C = oracle.cost_matrix(X, Y)
    # the oracle's potentials after 20 iterations, rounded to fp32, for both sides
    f32, g32 = (v.astype(np.float32) for v in oracle.sinkhorn(C, a, b, eps, 20))
    f = torch.from_numpy(f32).to(DEV)
    g = torch.from_numpy(g32).to(DEV)
    fh, gh = f32.astype(np.float64), g32.astype(np.float64)
    P = oracle.plan(C, a, b, fh, gh, eps)
    rng = np.random.default_rng(n + m + d)
    V = rng.standard_normal((m, cols)).astype(np.float32)
    U = rng.standard_normal((n, cols)).astype(np.float32)
    Vt = torch.from_numpy(V).to(DEV)
    Ut = torch.from_numpy(U).to(DEV)
    if dtype == "bf16":
        Vt, Ut = Vt.to(torch.bfloat16), Ut.to(torch.bfloat16)
    r = torch.empty(n, dtype=torch.float32, device=DEV)
    c = torch.empty(m, dtype=torch.float32, device=DEV)
    pv = ssa.ot_apply_plan(prob, f, g, Vt, marg=r)
    ptu = ssa.ot_apply_plan(prob, f, g, Ut, flags=ssa.OT_TRANSPOSE, marg=c)
    bary = ssa.ot_apply_plan(prob, f, g, Vt, flags=ssa.OT_BARY)
    grad = ssa.ot_apply_plan(prob, f, g, flags=ssa.OT_GRAD)
    gy = ssa.ot_apply_plan(prob, f, g, flags=ssa.OT_GRAD | ssa.OT_TRANSPOSE)
    torch.cuda.synchronize()
    Vh, Uh = host64(Vt), host64(Ut)
    r_ref, c_ref = oracle.marginals(P)
    assert _rel(host64(pv), oracle.apply_plan(P, Vh)) <= PV_TOL
    assert _rel(host64(ptu), oracle.apply_plan_t(P, Uh)) <= PV_TOL
    assert _rel(host64(bary), oracle.barycentric(P, Vh)) <= PV_TOL
    assert _rel(host64(r), r_ref) <= PV_TOL
    assert _rel(host64(c), c_ref) <= PV_TOL
    g_ref = oracle.grad_x(X, Y, P)
    assert _rel(host64(grad), g_ref) <= 10 * PV_TOL
    gy_ref = oracle.grad_x(Y, X, P.T)
    assert _rel(host64(gy), gy_ref) <= 10 * PV_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_apply_plan_value_column_scales(dtype):
    """The fp16 value layout scales each value column by its own power of two:
    columns of size 1e-6, 1 and 1e6 next to each other, and an all-zero one,
    each come out to the fp32 gate relative to their own size."""
    n, m, d, eps = 150, 170, 64, 0.1
    base = "c3_d16_bf16" if dtype == "bf16" else "c3_d16_f32"
    data = workloads.make(base, n=n, m=m, d=d)
    prob = make_problem(data, eps=eps)
    X, Y, a, b = oracle_inputs(prob)
    C = oracle.cost_matrix(X, Y)
    f32, g32 = (v.astype(np.float32) for v in oracle.sinkhorn(C, a, b, eps, 20))
    P = oracle.plan(C, a, b, f32.astype(np.float64), g32.astype(np.float64), eps)
    rng = np.random.default_rng(5)
    V = rng.standard_normal((m, 4)) * np.array([1e-6, 1.0, 1e6, 0.0])
    Vt = torch.from_numpy(V.astype(np.float32)).to(DEV)
    if dtype == "bf16":
        Vt = Vt.to(torch.bfloat16)
    pv = ssa.ot_apply_plan(prob, torch.from_numpy(f32).to(DEV), torch.from_numpy(g32).to(DEV), Vt)
    torch.cuda.synchronize()
    ref = oracle.apply_plan(P, host64(Vt))
    out = host64(pv)
    for k in range(3):
        assert _rel(out[:, k], ref[:, k]) <= PV_TOL, k
    assert np.all(out[:, 3] == 0.0)


@pytest.mark.parametrize("d,cols", [(64, 20), (512, 20), (512, 64)])
def test_apply_plan_f32_values_on_bf16_points(d, cols):
    """fp32 values (hi and lo fp16 parts) with bf16 points: resident rows, and
    wide rows with one value block (fragments read into registers) or two
    (staged in LDS)."""
    n, m, eps = 150, 210, 0.1
    say(f"f32 values on bf16 points d={d} cols={cols}")
    data = workloads.make("c3_d16_bf16", n=n, m=m, d=d)
    prob = make_problem(data, eps=eps)
    X, Y, a, b = oracle_inputs(prob)
    C = oracle.cost_matrix(X, Y)
    f32, g32 = (v.astype(np.float32) for v in oracle.sinkhorn(C, a, b, eps, 20))
    P = oracle.plan(C, a, b, f32.astype(np.float64), g32.astype(np.float64), eps)
    f, g = torch.from_numpy(f32).to(DEV), torch.from_numpy(g32).to(DEV)
    rng = np.random.default_rng(d + cols)
    V = rng.standard_normal((m, cols)).astype(np.float32)
    U = rng.standard_normal((n, cols)).astype(np.float32)
    pv = ssa.ot_apply_plan(prob, f, g, torch.from_numpy(V).to(DEV))
    ptu = ssa.ot_apply_plan(prob, f, g, torch.from_numpy(U).to(DEV), flags=ssa.OT_TRANSPOSE)
    torch.cuda.synchronize()
    assert _rel(host64(pv), oracle.apply_plan(P, V.astype(np.float64))) <= PV_TOL
    assert _rel(host64(ptu), oracle.apply_plan_t(P, U.astype(np.float64))) <= PV_TOL


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 1024), ("bf16", 64), ("bf16", 512)])
def test_apply_plan_bf16_values_take_one_part(dtype, d):
    """bf16 values enter the value product by their fp16 hi parts alone (their
    lo parts in the layout are zero): the result equals, bitwise, that of the
    same values given as fp32 (hi and lo parts), and matches the oracle, for
    register-resident and wide rows, columns spanning twelve decades included."""
    n, m, eps = 170, 150, 0.1
    say(f"bf16 values dtype={dtype} d={d}")
    base = "c3_d16_bf16" if dtype == "bf16" else "c3_d16_f32"
    data = workloads.make(base, n=n, m=m, d=d)
    prob = make_problem(data, eps=eps)
    X, Y, a, b = oracle_inputs(prob)
    C = oracle.cost_matrix(X, Y)
    f32, g32 = (v.astype(np.float32) for v in oracle.sinkhorn(C, a, b, eps, 20))
    P = oracle.plan(C, a, b, f32.astype(np.float64), g32.astype(np.float64), eps)
    f, g = torch.from_numpy(f32).to(DEV), torch.from_numpy(g32).to(DEV)
    rng = np.random.default_rng(d)
    V = rng.standard_normal((m, 3))
    V[:, 1] *= 10.0 ** rng.uniform(-12, 0, m)
    V[:, 2] *= 3e-20
    U = rng.standard_normal((n, 40))
    for M, flags, ref_fn in ((V, 0, oracle.apply_plan), (U, ssa.OT_TRANSPOSE, oracle.apply_plan_t)):
        Mb = torch.from_numpy(M.astype(np.float32)).to(DEV).to(torch.bfloat16)
        one = ssa.ot_apply_plan(prob, f, g, Mb, flags=flags)
        two = ssa.ot_apply_plan(prob, f, g, Mb.float(), flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(one, two)
        ref = ref_fn(P, host64(Mb))
        out = host64(one)
        for k in range(M.shape[1]):
            assert _rel(out[:, k], ref[:, k]) <= PV_TOL, k


# --- execution properties ---------------------------------------------------------------

def test_deterministic_graph_eager_and_resume():
    """Bitwise: two runs agree; graph replay equals plain launches; k then k'
    iterations equal k + k' (the bias is rebuilt from the stored potential)."""
    data = workloads.make("c2", n=1500, m=1300)
    prob = make_problem(data)
    outs = []
    for use_graph in (True, True, False):
        f, g = zeros(1500), zeros(1300)
        ssa.ot_solve(prob, f, g, 23, use_graph=use_graph, want_info=False)
        outs.append((f.clone(), g.clone()))
    torch.cuda.synchronize()
    for f, g in outs[1:]:
        assert torch.equal(f, outs[0][0]) and torch.equal(g, outs[0][1])
    f, g = zeros(1500), zeros(1300)
    ssa.ot_solve(prob, f, g, 10, want_info=False)
    ssa.ot_solve(prob, f, g, 13, init_given=True, want_info=False)
    torch.cuda.synchronize()
    assert torch.equal(f, outs[0][0]) and torch.equal(g, outs[0][1])


@pytest.mark.parametrize("schedule", ["alternating", "symmetric"])
def test_graph_replays_match_eager_with_work_between(schedule):
    """The cached iteration graphs, replayed by four solves in a row on one
    workspace with eager launches of the library and of torch and host
    synchronizations between them, give the eager result bitwise every time
    (a replay that reused stale state from the previous one would differ)."""
    n, m, T = 1400, 1100, 37  # two replays of the 16-iteration graph + 5 single ones
    data = workloads.make("c2", n=n, m=m)
    prob = make_problem(data)
    ws = ssa.solve_workspace(prob, T)
    fe, ge = zeros(n), zeros(m)
    ssa.ot_solve(prob, fe, ge, T, use_graph=False, want_info=False, ws=ws, schedule=schedule)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        f, g = zeros(n), zeros(m)
        ssa.ot_solve(prob, f, g, T, want_info=False, ws=ws, schedule=schedule)
        torch.cuda.synchronize()
        assert torch.equal(f, fe) and torch.equal(g, ge), rep
        # eager work between replays: the library's own half-steps on the same
        # workspace, a torch reduction, and a host round trip
        f2, g2 = f.clone(), g.clone()
        ssa.ot_update_f(prob, g2, f2, ws=ws)
        ssa.ot_update_g(prob, f2, g2, ws=ws)
        scratch.mul_(1.0001).sum().item()
        torch.cuda.synchronize()


@pytest.mark.parametrize("shape,schedule", [((300, 200), "alternating"),
                                            ((1500, 1300), "alternating"),
                                            ((1500, 1300), "symmetric")])
def test_timed_solve_equals_untimed(shape, schedule):
    """Timing every log-sum-exp dispatch (events recorded by the dispatch
    itself) changes no output bit: the single-launch half-steps of small
    problems, the split passes, and both passes of the symmetric schedule."""
    n, m = shape
    data = workloads.make("c2", n=n, m=m)
    prob = make_problem(data)
    T = 9
    f0, g0 = zeros(n), zeros(m)
    ref = ssa.ot_solve(prob, f0, g0, T, schedule=schedule)
    f, g = zeros(n), zeros(m)
    info = ssa.ot_solve(prob, f, g, T, schedule=schedule, timing=True)
    torch.cuda.synchronize()
    assert torch.equal(f, f0) and torch.equal(g, g0)
    assert info["marg_err_row"] == ref["marg_err_row"]
    assert info["marg_err_col"] == ref["marg_err_col"]
    assert info["lse_launches"] == 2 * T and ref["lse_launches"] == 0
    per = info["lse_ms"] / info["lse_launches"]
    say(f"timed solve {n}x{m} {schedule}: {1e3 * per:.1f} us per log-sum-exp launch")
    assert 0.0 < per < 100.0


def test_constant_mode_drift_and_rest_of_error():
    """Potentials after 100 iterations (n = m = 2000, the 20000-point workload's
    distributions) against the fp64 oracle, split into the drift along the
    constant direction (f + k, g - k), which leaves the coupling unchanged and
    along which any rounding bias of the score arithmetic accumulates
    (eigenvalue 1), and the rest of the error. Measured on gfx950: drift
    3.3e-6, rest 4.0e-7; a bias instruction adding onto a nonzero accumulator
    (rounding biased by about -0.2 ulp) had drifted 6.6e-6."""
    say("constant-mode drift n=m=2000")
    data = workloads.make("c2", n=2000, m=2000)
    prob = make_problem(data)
    X, Y, a, b = oracle_inputs(prob)
    f, g = zeros(2000), zeros(2000)
    ssa.ot_solve(prob, f, g, 100, want_info=False)
    torch.cuda.synchronize()
    f_ref, g_ref = oracle.sinkhorn(oracle.cost_matrix(X, Y), a, b, data["w"].eps, 100)
    df = host64(f) - f_ref
    dg = host64(g) - g_ref
    drift = 0.5 * (df.mean() - dg.mean())
    rest = max(np.abs(df - df.mean()).max(), np.abs(dg - dg.mean()).max())
    say(f"  drift {drift:.2e}, rest {rest:.2e}")
    assert abs(drift) <= 5e-6
    assert rest <= 1e-6
    assert abs(df.mean() + dg.mean()) <= 1e-6  # the drift is along (1, -1)


def test_split_count_changes_only_rounding():
    """The ⊕ merge of partial (max, sum) pairs is exact (App. D.3): any split count
    gives the same potentials up to fp32 rounding."""
    data = workloads.make("c3_d128_f32", n=900, m=1100)
    prob = make_problem(data)
    ref = None
    for sf, sg in ((1, 1), (3, 5), (8, 8), (34, 28)):
        f, g = zeros(900), zeros(1100)
        info = ssa.ot_solve(prob, f, g, 15, splits_f=sf, splits_g=sg)
        torch.cuda.synchronize()
        say(f"splits {sf},{sg} -> used {info['splits_f']},{info['splits_g']}")
        if ref is None:
            ref = (host64(f), host64(g))
        else:
            assert np.abs(host64(f) - ref[0]).max() <= 2e-5
            assert np.abs(host64(g) - ref[1]).max() <= 2e-5


# (n, m, d, dtype, waves per workgroup)
SOLO_CASES = [(1000, 700, 16, "f32", 4), (64, 100, 64, "f32", 4), (33, 1, 5, "bf16", 4),
              (1024, 1024, 128, "bf16", 4), (2048, 2048, 16, "f32", 4), (300, 2000, 32, "f32", 4)]


@pytest.mark.parametrize("n,m,d,dtype,waves", SOLO_CASES)
def test_single_launch_half_step_matches_split_path(n, m, d, dtype, waves):
    """Small problems run each half-step as one launch: the workgroup's waves
    split the columns and their (max, sum) pairs are merged on chip (App. D.3)
    before the potential is written. Against the oracle that is the same
    iteration; against the split pass + merge it differs only by the merge
    order's rounding. Waves past the last column tile (m = 1) contribute
    nothing."""
    data = workloads.make("c3_d16_f32", n=n, m=m, d=d)
    prob = make_problem(data, dtype=dtype)
    T = 20
    f, g = zeros(n), zeros(m)
    info = ssa.ot_solve(prob, f, g, T, want_info=True)
    f2, g2 = zeros(n), zeros(m)
    info2 = ssa.ot_solve(prob, f2, g2, T, splits_f=1, splits_g=1, want_info=True)
    torch.cuda.synchronize()
    ctiles = (m + 31) // 32
    tpw = (ctiles + waves - 1) // waves  # column tiles per wave
    say(f"single launch {n}x{m} d={d} {dtype}: splits used {info['splits_f']},{info['splits_g']} "
        f"(forced path {info2['splits_f']},{info2['splits_g']})")
    assert info["splits_f"] == (ctiles + tpw - 1) // tpw
    df = np.abs(host64(f) - host64(f2)).max()
    dg = np.abs(host64(g) - host64(g2)).max()
    say(f"  vs split path: max|df|={df:.2e} max|dg|={dg:.2e}")
    assert df <= 5e-5 and dg <= 5e-5
    X, Y, a, b = oracle_inputs(prob)
    f_ref, g_ref = oracle.sinkhorn(oracle.cost_matrix(X, Y), a, b, float(data["w"].eps), T)
    ef = np.abs(host64(f) - f_ref).max()
    eg = np.abs(host64(g) - g_ref).max()
    say(f"  vs oracle: max|df|={ef:.2e} max|dg|={eg:.2e}")
    assert ef <= POT_TOL["f32"] and eg <= POT_TOL["f32"]
    e1, e2 = info["marg_err_row"], info2["marg_err_row"]
    assert abs(e1 - e2) <= 1e-2 * max(e1, e2) + 1e-6


def test_tolerance_stops_early():
    data = workloads.make("c1", n=400, m=300)
    prob = make_problem(data)
    f, g = zeros(400), zeros(300)
    info = ssa.ot_solve(prob, f, g, 500, tol=1e-3, check_every=5)
    torch.cuda.synchronize()
    assert info["iters_done"] < 500 and info["iters_done"] % 5 == 0
    assert info["marg_err_row"] < 1e-3


def test_single_target_point_closed_form():
    """m = 1: f_i = C_i1 - g_1 - eps log b_1 and P V = a V_1^T (oracle pin, on the GPU)."""
    data = workloads.make("c3_d16_f32", n=77, m=1, d=5)
    prob = make_problem(data, weights=False)
    f, g = zeros(77), zeros(1)
    ssa.ot_solve(prob, f, g, 3, want_info=False)
    V = torch.from_numpy(np.random.default_rng(11).standard_normal((1, 4)).astype(np.float32)).to(DEV)
    pv = ssa.ot_apply_plan(prob, f, g, V)
    torch.cuda.synchronize()
    X, Y, a, b = oracle_inputs(prob)
    # P V gate (1e-4): P_i1 = a_i exp(rounding of f_i/eps), and f_i carries fp32
    # rounding of order ulp(|f|), amplified by 1/eps.
    np.testing.assert_allclose(host64(pv), a[:, None] * host64(V)[0][None, :], rtol=PV_TOL, atol=1e-9)
    assert abs(host64(g)[0]) < 1e-5


def test_nonfinite_reported():
    """A NaN weight propagates to the potentials; ot_solve with info says so."""
    data = workloads.make("c1", n=100, m=90)
    data["a"][5] = np.nan
    prob = make_problem(data)
    f, g = zeros(100), zeros(90)
    with pytest.raises(ssa.OtError) as ei:
        ssa.ot_solve(prob, f, g, 3)
    assert ei.value.code == ssa.OT_ERR_NONFINITE


@pytest.mark.parametrize("scale_exp", [-12, 8])
def test_half2_balances_point_scales(scale_exp):
    """The two-part fp16 operands take X and Y to the fp16 range by exact powers
    of two. Clouds scaled by s = 2^k with eps scaled by s^2 have potentials
    scaled by s^2; at k = -12 the unbalanced low parts would be fp16
    subnormals, at k = 8 the scaled X would be far from Y's magnitude. The
    returned potentials match the oracle's on the scaled inputs to the fp32
    gate times s^2."""
    s = 2.0 ** scale_exp
    data = workloads.make("c2", n=300, m=260)
    data["X"] = (data["X"] * s).astype(np.float32)
    data["Y"] = (data["Y"] * s).astype(np.float32)
    eps = float(np.float32(0.1 * s * s))
    say(f"half2 scale 2^{scale_exp} eps={eps}")
    prob = make_problem(data, eps=eps)
    X, Y, a, b = oracle_inputs(prob)
    f, g = zeros(300), zeros(260)
    info = ssa.ot_solve(prob, f, g, 20)
    torch.cuda.synchronize()
    assert info["operand_mode"] == 3
    f_ref, g_ref = oracle.sinkhorn(oracle.cost_matrix(X, Y), a, b, float(np.float32(eps)), 20)
    assert np.abs(host64(f) - f_ref).max() <= POT_TOL["f32"] * s * s
    assert np.abs(host64(g) - g_ref).max() <= POT_TOL["f32"] * s * s


def test_half2_range_exceeded_reported():
    """Coordinates too large for the two-part fp16 scores ((2/eps) log2(e)
    max|x| max|y| far above 2^30): every entry point that forms scores from
    fp32 points in the default mode returns OT_ERR_UNSUPPORTED before
    enqueuing its passes (outputs untouched), with or without an info struct;
    the three-part bf16 split covers the fp32 range."""
    data = workloads.make("c1", n=100, m=90)
    data["X"] = (data["X"] * 1e5).astype(np.float32)
    data["Y"] = (data["Y"] * 1e5).astype(np.float32)
    prob = make_problem(data, eps=1.0)
    V = dev(np.ones((90, 3), dtype=np.float32))
    U = dev(np.ones((100, 3), dtype=np.float32))

    def refused(call, *outs):
        marks = [o.fill_(7.0) for o in outs]
        with pytest.raises(ssa.OtError) as ei:
            call()
        torch.cuda.synchronize()
        assert ei.value.code == ssa.OT_ERR_UNSUPPORTED
        for o in marks:
            assert bool((o == 7.0).all()), "a refused call must not write its outputs"

    f, g = zeros(100), zeros(90)
    refused(lambda: ssa.ot_solve(prob, f, g, 3), f, g)
    refused(lambda: ssa.ot_solve(prob, f, g, 3, want_info=False), f, g)
    refused(lambda: ssa.ot_solve(prob, f, g, 3, use_graph=False, want_info=False), f, g)
    refused(lambda: ssa.ot_update_f(prob, g, f), f)
    refused(lambda: ssa.ot_update_g(prob, f, g), g)
    out = torch.empty((100, 3), device=DEV)
    refused(lambda: ssa.ot_apply_plan(prob, f, g, V, out=out), out)
    outg = torch.empty((100, 16), device=DEV)
    refused(lambda: ssa.ot_apply_plan(prob, f, g, flags=ssa.OT_GRAD, out=outg), outg)
    outt = torch.empty((90, 3), device=DEV)
    refused(lambda: ssa.ot_apply_plan(prob, f, g, U, flags=ssa.OT_TRANSPOSE, out=outt), outt)
    prob = make_problem(data, eps=1.0, mode="split_bf16")
    f, g = zeros(100), zeros(90)
    info = ssa.ot_solve(prob, f, g, 3)
    torch.cuda.synchronize()
    assert info["operand_mode"] == 2 and not info["nonfinite"]
    assert torch.isfinite(f).all() and torch.isfinite(g).all()


def test_bf16_points_at_extreme_scale_stay_finite():
    """bf16 points scaled by 1e5 at eps = 1 (scores near 2^34 in dot-product
    units, where fp32 resolves them only to thousands): the exact path's
    exponents are taken against the maximum of the rounded scores, so no row
    sum overflows or empties; potentials stay finite."""
    data = workloads.make("c1", n=100, m=90)
    data["X"] = (data["X"] * 1e5).astype(np.float32)
    data["Y"] = (data["Y"] * 1e5).astype(np.float32)
    prob = make_problem(data, eps=1.0, dtype="bf16")
    f, g = zeros(100), zeros(90)
    info = ssa.ot_solve(prob, f, g, 3)
    torch.cuda.synchronize()
    assert info["operand_mode"] == 1 and not info["nonfinite"]
    assert torch.isfinite(f).all() and torch.isfinite(g).all()


# --- size edges -------------------------------------------------------------------------

@pytest.mark.parametrize("d,dtype", [(8192, "f32"), (8192, "bf16"), (4097, "f32")])
def test_largest_dimension(d, dtype):
    """d at OT_MAX_D (and one past a power of two): the wide pass with its
    longest k-loop, split and bf16 operands; half-steps against the oracle."""
    say(f"largest d={d} {dtype}")
    n, m, eps = 70, 45, 0.1
    data = workloads.make("c3_d16_bf16" if dtype == "bf16" else "c3_d16_f32", n=n, m=m, d=d)
    prob = make_problem(data, eps=eps)
    X, Y, a, b = oracle_inputs(prob)
    C = oracle.cost_matrix(X, Y)
    g0 = (np.random.default_rng(d).standard_normal(m) * 0.3).astype(np.float32)
    f = zeros(n)
    ssa.ot_update_f(prob, torch.from_numpy(g0).to(DEV), f)
    torch.cuda.synchronize()
    f_ref = oracle.update_f(C, g0.astype(np.float64), b, eps)
    assert np.abs(host64(f) - f_ref).max() <= POT_TOL[dtype]
    # and a short trajectory
    f, g = zeros(n), zeros(m)
    ssa.ot_solve(prob, f, g, 10, want_info=False)
    torch.cuda.synchronize()
    f_ref, g_ref = oracle.sinkhorn(C, a, b, eps, 10)
    assert np.abs(host64(f) - f_ref).max() <= POT_TOL[dtype]
    assert np.abs(host64(g) - g_ref).max() <= POT_TOL[dtype]


def test_one_point_each_side():
    """n = m = 1: a single pair; the potentials match the oracle's and stay finite."""
    data = workloads.make("c3_d16_f32", n=1, m=1, d=7)
    prob = make_problem(data)
    X, Y, a, b = oracle_inputs(prob)
    f, g = zeros(1), zeros(1)
    info = ssa.ot_solve(prob, f, g, 5)
    torch.cuda.synchronize()
    C = oracle.cost_matrix(X, Y)
    f_ref, g_ref = oracle.sinkhorn(C, a, b, 0.1, 5)
    assert abs(float(host64(f)[0]) - f_ref[0]) <= POT_TOL["f32"]
    assert abs(float(host64(g)[0]) - g_ref[0]) <= POT_TOL["f32"]
    assert not info["nonfinite"]
