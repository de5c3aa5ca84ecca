"""Write fp64 oracle potentials after T alternating iterations at full benchmark shape.

TEST INFRASTRUCTURE: this script calls only ``oracle/`` (and the seeded input
generators of ``workloads``); nothing of the HIP path. Its outputs are the
stored expected values of ``tests/test_gpu_fullsize_solve.py``.

What it computes is ``oracle.sinkhorn(C, a, b, eps, T)`` from zero potentials
for the workload's own seeded inputs ("FlashSinkhorn: IO-Aware Entropic
Optimal Transport on GPU", §3.1 alternating updates, §4.1 / App. H.2 fixed
iteration count from f = g = 0), followed by the L1 marginal errors of the
final coupling (§2.2, App. E.1); with ``--schedule symmetric``,
``oracle.sinkhorn_symmetric`` (§3.1 symmetric updates, both half-steps from
the previous iterate, then averaged) into ``<name>_symmetric.npz``. The page compares its fp32 results with an
fp64 dense reference at benchmark sizes (§4.1 "Low-eps regime", Table 20);
this is that reference for the five workloads.

The full n x m cost does not fit one numpy call's temporaries at these sizes,
so the oracle's own functions are applied to slices, over forked worker
processes:

* the cost is ``oracle.cost_matrix`` of row slices of X against all of Y
  (the direct difference), stored once in a file-backed array;
* an f half-step is ``oracle.update_f`` on row slices C[r0:r1, :] -- every
  row's log-sum-exp runs over its whole row, so each f_i is bitwise the value
  the dense call gives;
* a g half-step is ``oracle.update_g`` on column slices C[:, c0:c1], each g_j
  over its whole column, likewise bitwise the dense value;
* the marginals r = P 1 and c = P^T 1 of the final coupling come from
  ``oracle.plan`` on row slices (r) and column slices (c).

``tests/test_golden_fullsize_script.py`` checks on a small workload that this
equals the dense ``oracle.sinkhorn`` bitwise.

Usage: python tests/golden/make_fullsize.py c2 c5 ... [--workers K] [--scratch DIR] [--resume]
       [--schedule symmetric]
Each workload writes ``tests/golden/fullsize/<name>.npz`` (f, g as float64 and
the marginal errors). The scratch folder holds the cached cost (up to 39 GB
for the 70000-point workload) and a checkpoint of (f, g) every 10
iterations; it is deleted afterwards. ``--resume`` continues an interrupted
run from that folder: the cached cost is kept once sampled rows of it,
recomputed, match it bitwise, and the iterations restart from the last
checkpoint (the half-steps are deterministic, so the result is the one an
uninterrupted run gives).
"""

from __future__ import annotations

import argparse
import multiprocessing as mp
import os
import shutil
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT_DIR = os.path.join(HERE, "fullsize")
BLOCK_ELEMS = 1 << 22          # elements of C per worker task

# State shared with the forked workers (set before the pool forks).
_S: dict = {}


def _cost_task(r):
    r0, r1 = r
    _S["C"][r0:r1] = oracle.cost_matrix(_S["X"][r0:r1], _S["Y"])
    return r1 - r0


def _f_task(r):
    r0, r1 = r
    _S["F"][r0:r1] = oracle.update_f(_S["C"][r0:r1], _S["G"], _S["b"], _S["eps"])
    return 0


def _g_task(c):
    c0, c1 = c
    _S["G"][c0:c1] = oracle.update_g(_S["C"][:, c0:c1], _S["F"], _S["a"], _S["eps"])
    return 0


# Symmetric schedule: both half-steps read the previous iterate (into FT, GT),
# then each potential is averaged with its half-step in the parent process.
def _ft_task(r):
    r0, r1 = r
    _S["FT"][r0:r1] = oracle.update_f(_S["C"][r0:r1], _S["G"], _S["b"], _S["eps"])
    return 0


def _gt_task(c):
    c0, c1 = c
    _S["GT"][c0:c1] = oracle.update_g(_S["C"][:, c0:c1], _S["F"], _S["a"], _S["eps"])
    return 0


def _r_task(r):
    r0, r1 = r
    P = oracle.plan(_S["C"][r0:r1], _S["a"][r0:r1], _S["b"], _S["F"][r0:r1], _S["G"], _S["eps"])
    return r0, P.sum(axis=1)


def _c_task(c):
    c0, c1 = c
    P = oracle.plan(_S["C"][:, c0:c1], _S["a"], _S["b"][c0:c1], _S["F"], _S["G"][c0:c1], _S["eps"])
    return c0, P.sum(axis=0)


def _ranges(count, step):
    return [(i, min(count, i + step)) for i in range(0, count, step)]


def _init_worker(niceness):
    try:
        os.nice(niceness)
    except OSError:
        pass


def _cached_cost_valid(C, X, Y, rows):
    """Whether a cost file left by an earlier run holds this workload's cost:
    first, middle and last row slices recomputed and compared bitwise."""
    picks = [rows[0], rows[len(rows) // 2], rows[-1]]
    return all(np.array_equal(C[r0:r1], oracle.cost_matrix(X[r0:r1], Y)) for r0, r1 in picks)


def solve_sliced(X, Y, a, b, eps, iters, workers, scratch, log=print, resume=False,
                 schedule="alternating"):
    """``oracle.sinkhorn`` from zero potentials, evaluated on row / column slices
    (``oracle.sinkhorn_symmetric`` with ``schedule="symmetric"``).

    Returns (f, g, err_row, err_col) with the L1 marginal errors of the final
    coupling. X, Y, a, b are the exact values the GPU receives (float32 or
    bf16-representable float32), widened to float64 here.
    """
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n, m = X.shape[0], Y.shape[0]
    os.makedirs(scratch, exist_ok=True)
    cpath = os.path.join(scratch, "cost.f64")
    ckpt = os.path.join(scratch, "checkpoint.npz")
    rows = _ranges(n, max(1, BLOCK_ELEMS // m))
    cols = _ranges(m, max(1, BLOCK_ELEMS // n))
    # cost rows: the direct difference materialises rows x m x d temporaries
    cost_rows = _ranges(n, max(1, (BLOCK_ELEMS * 4) // (m * max(1, X.shape[1]))))
    reuse = (resume and os.path.exists(cpath) and os.path.getsize(cpath) == n * m * 8)
    C = np.memmap(cpath, dtype=np.float64, mode="r+" if reuse else "w+", shape=(n, m))
    if reuse and not _cached_cost_valid(C, X, Y, cost_rows):
        log("  cached cost does not match this workload: recomputing it")
        reuse = False
    F = np.memmap(os.path.join(scratch, "f.f64"), dtype=np.float64, mode="w+", shape=(n,))
    G = np.memmap(os.path.join(scratch, "g.f64"), dtype=np.float64, mode="w+", shape=(m,))
    F[:] = 0.0
    G[:] = 0.0
    sym = schedule == "symmetric"
    if sym:
        FT = np.memmap(os.path.join(scratch, "ft.f64"), dtype=np.float64, mode="w+", shape=(n,))
        GT = np.memmap(os.path.join(scratch, "gt.f64"), dtype=np.float64, mode="w+", shape=(m,))
        _S.update(FT=FT, GT=GT)
    start = 0
    if reuse and os.path.exists(ckpt):
        with np.load(ckpt) as z:
            if int(z["iters"]) == int(iters) and z["f"].shape == (n,) and z["g"].shape == (m,):
                start = int(z["t"])
                F[:] = z["f"]
                G[:] = z["g"]
    _S.update(C=C, F=F, G=G, X=X, Y=Y, a=a, b=b, eps=float(eps))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_init_worker, initargs=(10,)) as pool:
        if reuse:
            log(f"  cost {n}x{m}: reused from {cpath}; from iteration {start}")
        else:
            for _ in pool.imap_unordered(_cost_task, cost_rows, chunksize=4):
                pass
            log(f"  cost {n}x{m}: {time.perf_counter() - t0:.1f} s")
        for t in range(start, int(iters)):
            if sym:
                for _ in pool.imap_unordered(_ft_task, rows):
                    pass
                for _ in pool.imap_unordered(_gt_task, cols):
                    pass
                F[:] = 0.5 * (np.asarray(F) + np.asarray(FT))
                G[:] = 0.5 * (np.asarray(G) + np.asarray(GT))
            else:
                for _ in pool.imap_unordered(_f_task, rows):
                    pass
                for _ in pool.imap_unordered(_g_task, cols):
                    pass
            if t % 10 == 9 or t == iters - 1:
                log(f"  iteration {t + 1}/{iters}: {time.perf_counter() - t0:.1f} s")
                tmp = ckpt + ".tmp.npz"
                np.savez(tmp, t=t + 1, iters=int(iters), f=np.array(F), g=np.array(G))
                os.replace(tmp, ckpt)
        r = np.empty(n)
        c = np.empty(m)
        for r0, v in pool.imap_unordered(_r_task, rows):
            r[r0:r0 + len(v)] = v
        for c0, v in pool.imap_unordered(_c_task, cols):
            c[c0:c0 + len(v)] = v
    f = np.array(F)
    g = np.array(G)
    _S.clear()
    del C, F, G
    if sym:
        del FT, GT
    shutil.rmtree(scratch, ignore_errors=True)
    return f, g, float(np.abs(r - a).sum()), float(np.abs(c - b).sum())


def make_one(name, workers, scratch, log=print, resume=False, schedule="alternating"):
    data = workloads.make(name)
    w = data["w"]
    tag = name if schedule == "alternating" else f"{name}_{schedule}"
    log(f"{tag}: n={w.n} m={w.m} d={w.d} {w.dtype} eps={w.eps} T={w.iters}, {workers} workers")
    t0 = time.perf_counter()
    f, g, er, ec = solve_sliced(data["X"], data["Y"], data["a"], data["b"], w.eps, w.iters,
                                workers, os.path.join(scratch, tag), log=log, resume=resume,
                                schedule=schedule)
    os.makedirs(OUT_DIR, exist_ok=True)
    path = os.path.join(OUT_DIR, f"{tag}.npz")
    np.savez_compressed(path, f=f, g=g, marg_err_row=er, marg_err_col=ec,
                        n=w.n, m=w.m, d=w.d, eps=w.eps, iters=w.iters, dtype=w.dtype,
                        schedule=schedule)
    log(f"{tag}: wrote {path} in {time.perf_counter() - t0:.0f} s; "
        f"marginal errors row {er:.3e} col {ec:.3e}")
    return path


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("names", nargs="+", help="workload names (workloads.WORKLOADS)")
    ap.add_argument("--workers", type=int, default=max(1, (os.cpu_count() or 2) - 1))
    ap.add_argument("--scratch", default=os.path.join(ROOT, ".golden_scratch"))
    ap.add_argument("--resume", action="store_true",
                    help="reuse the scratch folder of an interrupted run")
    ap.add_argument("--schedule", default="alternating", choices=["alternating", "symmetric"],
                    help="symmetric: writes <name>_symmetric.npz")
    args = ap.parse_args(argv)
    for name in args.names:
        if name not in workloads.WORKLOADS:
            raise SystemExit(f"unknown workload {name}")
        make_one(name, args.workers, args.scratch, log=lambda s: print(s, flush=True),
                 resume=args.resume, schedule=args.schedule)


if __name__ == "__main__":
    main()
