"""The full-shape reference script computes the dense oracle's iteration, and
its stored files match the workloads they name (no GPU).

``tests/golden/make_fullsize.py`` evaluates ``oracle.sinkhorn`` on row and
column slices over worker processes. Each f_i is a log-sum-exp over its whole
row and each g_j over its whole column, so the result must equal the dense
call bitwise; a slicing mistake (a wrong slice bound, a transposed block, a
half-step reading a stale potential) would show here.
"""

import os
import sys

import numpy as np
import pytest

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_fullsize  # noqa: E402


@pytest.mark.parametrize("n,m,d,iters,workers", [(130, 97, 5, 7, 3), (64, 200, 17, 4, 2)])
def test_sliced_solve_equals_dense_oracle(tmp_path, n, m, d, iters, workers, monkeypatch):
    data = workloads.make("c3_d16_f32", n=n, m=m, d=d)
    eps = 0.07
    # small slices, so that every half-step spans several tasks
    monkeypatch.setattr(make_fullsize, "BLOCK_ELEMS", 1000)
    f, g, er, ec = make_fullsize.solve_sliced(data["X"], data["Y"], data["a"], data["b"], eps,
                                             iters, workers, str(tmp_path / "scratch"))
    X, Y = data["X"].astype(np.float64), data["Y"].astype(np.float64)
    a, b = data["a"].astype(np.float64), data["b"].astype(np.float64)
    C = oracle.cost_matrix(X, Y)
    f_ref, g_ref = oracle.sinkhorn(C, a, b, eps, iters)
    assert np.array_equal(f, f_ref) and np.array_equal(g, g_ref)
    er_ref, ec_ref = oracle.marginal_errors(oracle.plan(C, a, b, f_ref, g_ref, eps), a, b)
    assert er == pytest.approx(er_ref, rel=1e-12, abs=1e-300)
    assert ec == pytest.approx(ec_ref, rel=1e-9, abs=1e-15)
    assert not os.path.exists(tmp_path / "scratch")


def test_sliced_symmetric_solve_equals_dense_oracle(tmp_path, monkeypatch):
    """The symmetric schedule (both half-steps from the previous iterate, then
    averaged) sliced over workers equals ``oracle.sinkhorn_symmetric`` bitwise."""
    n, m, d, eps, iters = 110, 85, 7, 0.09, 6
    data = workloads.make("c3_d16_f32", n=n, m=m, d=d)
    monkeypatch.setattr(make_fullsize, "BLOCK_ELEMS", 1000)
    f, g, er, ec = make_fullsize.solve_sliced(data["X"], data["Y"], data["a"], data["b"], eps,
                                             iters, 3, str(tmp_path / "scratch"),
                                             schedule="symmetric")
    X, Y = data["X"].astype(np.float64), data["Y"].astype(np.float64)
    a, b = data["a"].astype(np.float64), data["b"].astype(np.float64)
    C = oracle.cost_matrix(X, Y)
    f_ref, g_ref = oracle.sinkhorn_symmetric(C, a, b, eps, iters)
    assert np.array_equal(f, f_ref) and np.array_equal(g, g_ref)
    er_ref, ec_ref = oracle.marginal_errors(oracle.plan(C, a, b, f_ref, g_ref, eps), a, b)
    assert er == pytest.approx(er_ref, rel=1e-12) and ec == pytest.approx(ec_ref, rel=1e-12)


def test_resumed_run_equals_dense_oracle(tmp_path, monkeypatch):
    """An interrupted run resumed from its scratch folder (cached cost, a
    checkpoint of (f, g) after 10 of 20 iterations) ends where the dense
    iteration does, bitwise; a cost file of another workload is recomputed."""
    n, m, d, eps, iters = 90, 70, 6, 0.08, 20
    data = workloads.make("c3_d16_f32", n=n, m=m, d=d)
    monkeypatch.setattr(make_fullsize, "BLOCK_ELEMS", 1000)
    X, Y = data["X"].astype(np.float64), data["Y"].astype(np.float64)
    a, b = data["a"].astype(np.float64), data["b"].astype(np.float64)
    C = oracle.cost_matrix(X, Y)
    scratch = tmp_path / "scratch"
    scratch.mkdir()
    f10, g10 = oracle.sinkhorn(C, a, b, eps, 10)
    np.savez(scratch / "checkpoint.npz", t=10, iters=iters, f=f10, g=g10)
    C.tofile(scratch / "cost.f64")
    f, g, _, _ = make_fullsize.solve_sliced(data["X"], data["Y"], data["a"], data["b"], eps,
                                           iters, 2, str(scratch), resume=True)
    f_ref, g_ref = oracle.sinkhorn(C, a, b, eps, iters)
    assert np.array_equal(f, f_ref) and np.array_equal(g, g_ref)
    # a cost file that is not this workload's is not trusted
    scratch.mkdir()
    np.savez(scratch / "checkpoint.npz", t=10, iters=iters, f=f10, g=g10)
    (C + 1.0).tofile(scratch / "cost.f64")
    f, g, _, _ = make_fullsize.solve_sliced(data["X"], data["Y"], data["a"], data["b"], eps,
                                           iters, 2, str(scratch), resume=True)
    assert np.array_equal(f, f_ref) and np.array_equal(g, g_ref)


def test_stored_references_describe_their_workloads():
    gold = os.path.join(HERE, "golden", "fullsize")
    names = sorted(fn[:-4] for fn in os.listdir(gold) if fn.endswith(".npz")) if os.path.isdir(gold) else []
    assert "c2" in names, "the headline workload's reference potentials are committed"
    for name in names:
        z = np.load(os.path.join(gold, f"{name}.npz"))
        sym = name.endswith("_symmetric")
        w = workloads.WORKLOADS[name[:-len("_symmetric")] if sym else name]
        assert str(z["schedule"]) == ("symmetric" if sym else "alternating") if "schedule" in z \
            else not sym
        assert (int(z["n"]), int(z["m"]), int(z["d"]), int(z["iters"])) == (w.n, w.m, w.d, w.iters)
        assert float(z["eps"]) == w.eps and str(z["dtype"]) == w.dtype
        assert z["f"].shape == (w.n,) and z["g"].shape == (w.m,)
        assert np.all(np.isfinite(z["f"])) and np.all(np.isfinite(z["g"]))
        if not sym:
            # after a g half-step the column marginal is met to fp64 rounding
            assert float(z["marg_err_col"]) < 1e-9
