"""ot_solve_static (the entry point for callers that cannot allocate) against
ot_solve with a caller workspace, through the C ABI.

Both run the same kernels on the same packed layout; ot_solve_static takes
its workspace from the library's static device scratch and launches plainly
(no graph). The kernels are deterministic and the alternating iterations are
bitwise the same with and without graph replay, so the potentials and the
reported marginal errors must agree exactly -- stricter than the 1e-4 (fp32)
/ 2e-2 (bf16) parity bar. Two calls in a row, the second on a smaller problem
(the scratch keeps the first call's contents), then one that needs more
scratch than the static array holds, which must be refused before any work.
"""

import ctypes

import numpy as np
import pytest
import torch

import streaming_sinkhorn_amd as ssa
import workloads
from gpu_util import make_problem, say, zeros


@pytest.mark.gpu
def test_static_scratch_solve_matches_workspace_solve():
    for name, n, m, d, iters in (("c2", 3000, 2600, 64, 25), ("c3_d16_bf16", 900, 700, 16, 20)):
        data = workloads.make(name, n=n, m=m, d=d)
        w = data["w"]
        say(f"static-scratch solve {name} n={n} m={m} d={d} {w.dtype} iters={iters}")
        prob = make_problem(data)
        f1, g1 = zeros(n), zeros(m)
        i1 = ssa.ot_solve(prob, f1, g1, iters)
        f2, g2 = zeros(n), zeros(m)
        i2 = ssa.ot_solve_static(prob, f2, g2, iters)
        torch.cuda.synchronize()
        say(f"  max|df|={float((f1 - f2).abs().max()):.3e} max|dg|={float((g1 - g2).abs().max()):.3e}")
        assert torch.equal(f1, f2) and torch.equal(g1, g2)
        for k in ("iters_done", "nonfinite", "marg_err_row", "marg_err_col", "operand_mode",
                  "splits_f", "splits_g"):
            assert i1[k] == i2[k], k
        assert np.isfinite(i2["marg_err_row"]) and not i2["nonfinite"]


@pytest.mark.gpu
def test_static_scratch_refuses_oversized_problems():
    data = workloads.make("c2", n=64, m=64)
    prob = make_problem(data)
    need = ctypes.c_size_t(0)
    # an n x m x d whose workspace exceeds the scratch (same dtype and device pointers;
    # the call must fail on the size check before any launch)
    big = ssa.OtProblem(prob.c.x, prob.c.y, 400000, 400000, 512, 512, 512, prob.c.dtype, prob.c.eps,
                        None, None, None, None, 0)
    opts = ssa.OtSolveOpts(10, 0.0, 1, 0, 1, 0, 0, 0)
    L = ssa.lib()
    assert L.ot_solve(ctypes.byref(big), None, None, ctypes.byref(opts), None, None,
                      ctypes.byref(need), None) == ssa.OT_OK
    assert need.value > ssa.static_scratch_bytes()
    rc = L.ot_solve_static(ctypes.byref(big), None, None, ctypes.byref(opts), None, None)
    assert rc == ssa.OT_ERR_WORKSPACE
    assert b"static" in L.ot_last_error()
