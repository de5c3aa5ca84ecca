"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host before any HIP call
(workspace-size queries are host-only as well)."""

import ctypes
import os
import subprocess

import pytest

import streaming_sinkhorn_amd as ssa

LIB = ssa.LIB_PATH
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libflashot.so not built")


def _problem(n=100, m=70, d=16, dtype=ssa.OT_F32, eps=0.1, x=1 << 20, y=2 << 20):
    # Fake, never dereferenced device addresses: every call below fails or
    # returns during host-side validation / size queries.
    return ssa.OtProblem(x, y, n, m, d, d, d, dtype, eps, None, None, None, None)


def _size(fn, *args):
    sz = ctypes.c_size_t(0)
    rc = fn(*args, None, ctypes.byref(sz), None)
    return rc, sz.value


def test_exports_every_header_symbol():
    names = ssa.header_entry_points()
    assert set(["ot_sqnorms", "ot_update_f", "ot_update_g", "ot_solve", "ot_apply_plan"]) <= set(names)
    L = ssa.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, f"{n} not exported with C linkage"
    assert ssa.version().startswith("flashot")


def test_workspace_query_is_host_only_and_monotone():
    L = ssa.lib()
    p1 = _problem(1000, 1000, 64)
    p2 = _problem(2000, 1000, 64)
    rc1, s1 = _size(L.ot_update_f, ctypes.byref(p1), None, None, None)
    rc2, s2 = _size(L.ot_update_f, ctypes.byref(p2), None, None, None)
    assert rc1 == 0 and rc2 == 0 and 0 < s1 < s2
    opts = ssa.OtSolveOpts(10, 0.0, 1, 0, 1, 0, 0, 0)
    sz = ctypes.c_size_t(0)
    assert L.ot_solve(ctypes.byref(p1), None, None, ctypes.byref(opts), None, None, ctypes.byref(sz), None) == 0
    assert sz.value >= s1
    sz = ctypes.c_size_t(0)
    assert L.ot_apply_plan(ctypes.byref(p1), None, None, None, 0, 64, 64, 0, None, None, None,
                           ctypes.byref(sz), None) == 0
    assert sz.value > 0


@pytest.mark.parametrize("field,value,code", [
    ("n", 0, ssa.OT_ERR_INVALID_ARG),
    ("m", -3, ssa.OT_ERR_INVALID_ARG),
    ("d", 0, ssa.OT_ERR_INVALID_ARG),
    ("ldx", 8, ssa.OT_ERR_INVALID_ARG),
    ("eps", 0.0, ssa.OT_ERR_INVALID_ARG),
    ("eps", -1.0, ssa.OT_ERR_INVALID_ARG),
    ("eps", float("nan"), ssa.OT_ERR_INVALID_ARG),
    ("eps", 1e-45, ssa.OT_ERR_UNSUPPORTED),
    ("dtype", 7, ssa.OT_ERR_UNSUPPORTED),
    ("d", 100000, ssa.OT_ERR_UNSUPPORTED),
    ("x", 0, ssa.OT_ERR_INVALID_ARG),
    ("x", (1 << 20) + 2, ssa.OT_ERR_INVALID_ARG),   # fp32 data must be 4-byte aligned
    ("flags", 8, ssa.OT_ERR_INVALID_ARG),            # unknown problem flag
    ("flags", ssa.OT_COST_AFFINE, ssa.OT_ERR_INVALID_ARG),  # affine cost without alpha, beta
    ("flags", ssa.OT_NATIVE_F32 | ssa.OT_SPLIT_BF16, ssa.OT_ERR_INVALID_ARG),  # exclusive modes
])
def test_problem_validation(field, value, code):
    L = ssa.lib()
    p = _problem()
    setattr(p, field, value)
    if field == "d" and value > 16:
        p.ldx = p.ldy = value
    for fn in (L.ot_update_f, L.ot_update_g):
        rc, _ = _size(fn, ctypes.byref(p), None, None, None)
        assert rc == code, (field, value, rc, L.ot_last_error())
    assert L.ot_last_error()


def test_operand_mode_workspaces_differ():
    """fp32 points pack two fp16 parts per k-block by default (here d = 64:
    2 KiB per 16 values and 32 rows, as much as fp32 operands under
    OT_NATIVE_F32), three bf16 parts (3 KiB) under OT_SPLIT_BF16."""
    L = ssa.lib()
    p = _problem(1024, 1024, 64)
    _, half2 = _size(L.ot_update_f, ctypes.byref(p), None, None, None)
    p.flags = ssa.OT_NATIVE_F32
    _, native = _size(L.ot_update_f, ctypes.byref(p), None, None, None)
    p.flags = ssa.OT_SPLIT_BF16
    _, split = _size(L.ot_update_f, ctypes.byref(p), None, None, None)
    tiles = 1024 // 32
    assert half2 == native
    assert split - native == 2 * tiles * (3 * 4 - 8) * 1024
    p.flags = ssa.OT_SPLIT_BF16 | ssa.OT_NATIVE_F32
    rc, _ = _size(L.ot_update_f, ctypes.byref(p), None, None, None)
    assert rc == ssa.OT_ERR_INVALID_ARG and b"exclusive" in L.ot_last_error()


def test_null_problem_and_null_sizes():
    L = ssa.lib()
    assert L.ot_update_f(None, None, None, None, None, None, None) == ssa.OT_ERR_INVALID_ARG
    p = _problem()
    assert L.ot_update_f(ctypes.byref(p), None, None, None, None, None, None) == ssa.OT_ERR_INVALID_ARG
    assert L.ot_sqnorms(None, 0, 10, 4, 4, None, None) == ssa.OT_ERR_INVALID_ARG
    assert L.ot_sqnorms(1 << 20, 0, 0, 4, 4, 2 << 20, None) == ssa.OT_ERR_INVALID_ARG
    assert L.ot_sqnorms(1 << 20, 5, 10, 4, 4, 2 << 20, None) == ssa.OT_ERR_UNSUPPORTED


def test_workspace_too_small_and_misaligned():
    L = ssa.lib()
    p = _problem()
    rc, need = _size(L.ot_update_f, ctypes.byref(p), None, None, None)
    small = ctypes.c_size_t(need - 1)
    assert L.ot_update_f(ctypes.byref(p), 3 << 20, 4 << 20, None, 5 << 20, ctypes.byref(small), None) \
        == ssa.OT_ERR_WORKSPACE
    ok = ctypes.c_size_t(need)
    assert L.ot_update_f(ctypes.byref(p), 3 << 20, 4 << 20, None, (5 << 20) + 4, ctypes.byref(ok), None) \
        == ssa.OT_ERR_INVALID_ARG


def test_solve_option_validation():
    L = ssa.lib()
    p = _problem()
    sz = ctypes.c_size_t(1 << 40)
    bad = [
        ssa.OtSolveOpts(-1, 0.0, 1, 0, 1, 0, 0, 0),      # iters < 0
        ssa.OtSolveOpts(5, -1.0, 1, 0, 1, 0, 0, 0),      # tol < 0
        ssa.OtSolveOpts(5, 1e-3, 0, 0, 1, 0, 0, 0),      # tol > 0 needs check_every
        ssa.OtSolveOpts(5, 0.0, 1, 9, 1, 0, 0, 0),       # init
        ssa.OtSolveOpts(5, 0.0, 1, 0, 1, -2, 0, 0),      # splits
        ssa.OtSolveOpts(5, 0.0, 1, 0, 1, 0, 0, 1),       # timing without info
    ]
    for o in bad:
        assert L.ot_solve(ctypes.byref(p), 1 << 21, 1 << 22, ctypes.byref(o), None, 1 << 23,
                          ctypes.byref(sz), None) == ssa.OT_ERR_INVALID_ARG
    assert L.ot_solve(ctypes.byref(p), 1 << 21, 1 << 22, None, None, 1 << 23, ctypes.byref(sz), None) \
        == ssa.OT_ERR_INVALID_ARG


def test_solve_schedule_validation():
    L = ssa.lib()
    p = _problem()
    sz = ctypes.c_size_t(0)
    for sched, code in ((ssa.OT_SCHED_ALTERNATING, ssa.OT_OK), (ssa.OT_SCHED_SYMMETRIC, ssa.OT_OK),
                        (2, ssa.OT_ERR_INVALID_ARG), (-1, ssa.OT_ERR_INVALID_ARG)):
        opts = ssa.OtSolveOpts(5, 0.0, 1, 0, 1, 0, 0, 0, sched)
        assert L.ot_solve(ctypes.byref(p), None, None, ctypes.byref(opts), None, None,
                          ctypes.byref(sz), None) == code


def test_apply_plan_validation():
    L = ssa.lib()
    p = _problem()
    sz = ctypes.c_size_t(1 << 40)
    args = lambda v_dtype, cols, ldv, flags: L.ot_apply_plan(
        ctypes.byref(p), 1 << 21, 1 << 22, 1 << 23, v_dtype, cols, ldv, flags, 1 << 24, None,
        1 << 25, ctypes.byref(sz), None)
    assert args(0, 0, 0, 0) == ssa.OT_ERR_INVALID_ARG          # cols < 1
    assert args(0, 8, 4, 0) == ssa.OT_ERR_INVALID_ARG          # ldv < cols
    assert args(3, 8, 8, 0) == ssa.OT_ERR_UNSUPPORTED          # v dtype
    assert args(0, 8, 8, 64) == ssa.OT_ERR_INVALID_ARG         # unknown flag
    assert args(0, 8, 8, ssa.OT_GRAD | ssa.OT_BARY) == ssa.OT_ERR_INVALID_ARG
    assert args(0, 100000, 100000, 0) == ssa.OT_ERR_UNSUPPORTED


def test_binding_refuses_to_run_without_library(tmp_path, monkeypatch):
    """The product path has no fallback: a missing library raises on use."""
    monkeypatch.setattr(ssa, "_lib", None)
    monkeypatch.setattr(ssa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        ssa.lib()


# --- second-order entry points ------------------------------------------------------

def _hvp_size(p, opts, lda=16):
    L = ssa.lib()
    sz = ctypes.c_size_t(0)
    rc = L.ot_hvp(ctypes.byref(p), None, None, None, lda, None if opts is None else ctypes.byref(opts),
                  None, None, None, ctypes.byref(sz), None)
    return rc, sz.value


def test_hvp_and_hadamard_workspace_queries():
    L = ssa.lib()
    opts = ssa.OtHvpOpts(1e-5, 50, 0.0)
    rc1, s1 = _hvp_size(_problem(1000, 800, 16), opts)
    rc2, s2 = _hvp_size(_problem(2000, 800, 16), opts)
    assert rc1 == 0 and rc2 == 0 and 0 < s1 < s2
    sz = ctypes.c_size_t(0)
    assert L.ot_apply_hadamard(ctypes.byref(_problem(1000, 800, 16)), None, None, None, 16, None,
                               8, 8, None, None, ctypes.byref(sz), None) == 0
    assert 0 < sz.value < s1


@pytest.mark.parametrize("tau,iters,tol,code", [
    (-1e-5, 50, 0.0, ssa.OT_ERR_INVALID_ARG),
    (float("nan"), 50, 0.0, ssa.OT_ERR_INVALID_ARG),
    (float("inf"), 50, 0.0, ssa.OT_ERR_INVALID_ARG),
    (1e-5, -1, 0.0, ssa.OT_ERR_INVALID_ARG),
    (1e-5, 50, -1e-6, ssa.OT_ERR_INVALID_ARG),
    (1e-5, 50, float("nan"), ssa.OT_ERR_INVALID_ARG),
])
def test_hvp_option_validation(tau, iters, tol, code):
    rc, _ = _hvp_size(_problem(), ssa.OtHvpOpts(tau, iters, tol))
    assert rc == code, ssa.lib().ot_last_error()


def test_hvp_rejects_bf16_missing_opts_and_short_lda():
    L = ssa.lib()
    opts = ssa.OtHvpOpts(1e-5, 50, 0.0)
    rc, _ = _hvp_size(_problem(dtype=ssa.OT_BF16), opts)
    assert rc == ssa.OT_ERR_UNSUPPORTED
    rc, _ = _hvp_size(_problem(), None)
    assert rc == ssa.OT_ERR_INVALID_ARG
    # past the size query: null potentials, then a short lda, are rejected on the host
    p = _problem()
    sz = ctypes.c_size_t(1 << 40)
    fake = ctypes.c_void_p(1 << 24)
    rc = L.ot_hvp(ctypes.byref(p), None, None, None, 16, ctypes.byref(opts), None, None, fake,
                  ctypes.byref(sz), None)
    assert rc == ssa.OT_ERR_INVALID_ARG and "NULL" in L.ot_last_error().decode()
    rc = L.ot_hvp(ctypes.byref(p), fake, fake, fake, 15, ctypes.byref(opts), fake, None, fake,
                  ctypes.byref(sz), None)
    assert rc == ssa.OT_ERR_INVALID_ARG and "lda" in L.ot_last_error().decode()
    sz = ctypes.c_size_t(0)
    rc = L.ot_apply_hadamard(ctypes.byref(_problem(dtype=ssa.OT_BF16)), None, None, None, 16, None,
                             8, 8, None, None, ctypes.byref(sz), None)
    assert rc == ssa.OT_ERR_UNSUPPORTED
    rc = L.ot_apply_hadamard(ctypes.byref(_problem()), None, None, None, 16, None, 0, 8, None,
                             None, ctypes.byref(sz), None)
    assert rc == ssa.OT_ERR_INVALID_ARG


def test_affine_cost_rejected_where_the_cost_must_be_euclidean():
    L = ssa.lib()
    p = _problem()
    p.flags = ssa.OT_COST_AFFINE
    p.x_sqn, p.y_sqn = 3 << 20, 4 << 20   # alpha, beta given: the problem itself is valid
    rc, size = _size(L.ot_update_f, ctypes.byref(p), None, None, None)
    assert rc == 0 and size > 0
    sz = ctypes.c_size_t(0)
    rc = L.ot_apply_plan(ctypes.byref(p), None, None, None, 0, 16, 16, ssa.OT_GRAD, None, None, None,
                         ctypes.byref(sz), None)
    assert rc == ssa.OT_ERR_UNSUPPORTED
    rc, _ = _hvp_size(p, ssa.OtHvpOpts(1e-5, 50, 0.0))
    assert rc == ssa.OT_ERR_UNSUPPORTED


@pytest.mark.parametrize("args,code", [
    (dict(pts=None), ssa.OT_ERR_INVALID_ARG),
    (dict(rows=0), ssa.OT_ERR_INVALID_ARG),
    (dict(ld=3), ssa.OT_ERR_INVALID_ARG),
    (dict(dtype=5), ssa.OT_ERR_UNSUPPORTED),
    (dict(out=None), ssa.OT_ERR_INVALID_ARG),
    (dict(n_labels=0), ssa.OT_ERR_INVALID_ARG),
    (dict(side=2), ssa.OT_ERR_INVALID_ARG),
    (dict(d=8190), ssa.OT_ERR_UNSUPPORTED),
])
def test_prep_validation(args, code):
    L = ssa.lib()
    base = dict(pts=1 << 20, dtype=ssa.OT_F32, rows=10, d=4, ld=4, labels=2 << 20, W=3 << 20,
                n_labels=5, side=0, out=4 << 20, sqn=5 << 20)
    base.update(args)
    if base["d"] > 4:
        base["ld"] = base["d"]
    if "n_labels" not in args and "side" not in args and "d" not in args:
        rc = L.ot_prep_cosine(base["pts"], base["dtype"], base["rows"], base["d"], base["ld"],
                              base["out"], base["sqn"], None)
        assert rc == code, L.ot_last_error()
    rc = L.ot_prep_labels(base["pts"], base["dtype"], base["rows"], base["d"], base["ld"],
                          base["labels"], base["W"], base["n_labels"], base["side"], base["out"],
                          base["sqn"], None)
    assert rc == code, L.ot_last_error()


@pytest.mark.parametrize("eps_start,decay,code", [
    (-1.0, 0.5, ssa.OT_ERR_INVALID_ARG),
    (float("nan"), 0.5, ssa.OT_ERR_INVALID_ARG),
    (1.0, 0.0, ssa.OT_ERR_INVALID_ARG),
    (1.0, 1.0, ssa.OT_ERR_INVALID_ARG),
    (1.0, float("nan"), ssa.OT_ERR_INVALID_ARG),
    (0.05, 7.0, ssa.OT_OK),            # eps_start below eps: scaling off, decay unused
    (1.0, 0.5, ssa.OT_OK),
])
def test_eps_scaling_option_validation(eps_start, decay, code):
    L = ssa.lib()
    p = _problem(eps=0.1)
    opts = ssa._solve_opts(10, eps_start=eps_start, eps_decay=decay)
    sz = ctypes.c_size_t(0)
    rc = L.ot_solve(ctypes.byref(p), None, None, ctypes.byref(opts), None, None, ctypes.byref(sz), None)
    assert rc == code, L.ot_last_error()


def test_divergence_workspace_and_validation():
    L = ssa.lib()
    p = _problem(300, 200, 16)
    opts = ssa._solve_opts(10)
    sz = ctypes.c_size_t(0)
    assert L.ot_sinkhorn_divergence(ctypes.byref(p), ctypes.byref(opts), None, None, None, None, None,
                                    None, ctypes.byref(sz), None) == 0
    s_div = sz.value
    sz = ctypes.c_size_t(0)
    assert L.ot_solve(ctypes.byref(p), None, None, ctypes.byref(opts), None, None, ctypes.byref(sz),
                      None) == 0
    assert s_div >= sz.value + (300 + 200) * 4
    assert L.ot_sinkhorn_divergence(ctypes.byref(p), None, None, None, None, None, None, None,
                                    ctypes.byref(sz), None) == ssa.OT_ERR_INVALID_ARG
    p.flags = ssa.OT_COST_AFFINE
    p.x_sqn, p.y_sqn = 3 << 20, 4 << 20
    assert L.ot_sinkhorn_divergence(ctypes.byref(p), ctypes.byref(opts), None, None, None, None, None,
                                    None, ctypes.byref(sz), None) == ssa.OT_ERR_UNSUPPORTED


def test_solve_static_validates_on_the_host():
    """ot_solve_static (no workspace, no allocation) rejects a missing opts
    struct and a problem whose workspace exceeds its static scratch before
    any HIP call (fake device addresses, never dereferenced)."""
    L = ssa.lib()
    p = _problem(1000, 1000, 64)
    assert L.ot_solve_static(ctypes.byref(p), None, None, None, None, None) == ssa.OT_ERR_INVALID_ARG
    big = _problem(400000, 400000, 512)
    opts = ssa.OtSolveOpts(10, 0.0, 1, 0, 1, 0, 0, 0)
    assert L.ot_solve_static(ctypes.byref(big), None, None, ctypes.byref(opts), None, None) == ssa.OT_ERR_WORKSPACE
    assert ssa.static_scratch_bytes() == 64 << 20
