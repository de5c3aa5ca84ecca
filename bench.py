"""Throughput of the streamed Sinkhorn hot path on one MI355X.

A step is one pass of the whole path over one workload (default: the
n = m = 20000, d = 64 fp32 point clouds, eps = 0.1): squared norms of both
clouds, T alternating log-domain Sinkhorn iterations from zero potentials
(plain launches with a HIP event pair around every log-sum-exp kernel, on the
stream the kernels run on), the exact marginal errors of the returned
potentials, and the workload's transport applications (the P Y gradient for
the default workload; P V and P^T U where the workload has value matrices).
Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line. ``value`` = n * m * T / second of the whole step.
``roofline`` prices the dominant kernel (the streamed log-sum-exp pass) from
its average HIP-event duration inside the timed steps: against the dense
MFMA peak of the input type at 2 d flops per (i, j) pair, or -- when the
exponentials and vector work dominate (small d in bf16) -- against the ALU
bound of the online log-sum-exp in pairs per second. ``cpu_baseline`` times
the fp64 oracle on a bounded sample of the same workload on the host.

Without --graph the line also carries ``graph_replay``: the same steps with
the iterations replayed from HIP graphs (how ot_solve runs by default),
timed after the event-timed ones, for reference. Workloads of at most 4e8
pairs also report ``iteration_graph_us``: one iteration with graph replay,
from the difference of a 60- and a 20-iteration solve (the launch-bound
latency of small problems; not part of ``value``).

With --graph the timed steps replay the iterations from HIP graphs (no
per-launch events); the roofline then comes from one extra plain step.

Other modes:
  --gemm-probe       time torch.matmul (hipBLASLt) on random bf16 data at
                     16384^3 and 20000 x 1024 x 20000 and exit: the matrix
                     rate the chip sustains in a library GEMM, for context.
  --copy-probe MIB   copy a MIB-MiB buffer a few times with torch and exit:
                     the calibration run for the HBM byte counters.
  --exp-probe        time the library's throughput probes (v_exp_f32 and the
                     32x32x16 fp16 matrix instruction, include/flashot_probe.h)
                     and exit.

Roofline pricing: the method's own work per launch, 2 d flops and one
exponential per (i, j) pair, each against the published peak of the unit it
runs on (fp16 matrix cores for the default fp32 operands, which form every
fp32 product from two fp16 parts; bf16 for bf16 points and the three-part
split; fp32 for OT_NATIVE_F32; exponentials at EXP_PEAK_PER_S). The bound is
the larger of the two ideal times and frac = that time / the measured one.
``executed_frac`` gives the matrix work the kernel actually issues (three
products per fp32 product in the default mode) against the same peak.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks.
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0, "f16": 2500.0}
HBM_PEAK_GBS = 8000.0
# Exponential peak of the online log-sum-exp, from the unit counts: 256 CUs x
# 4 SIMDs x 8 lanes per clock x 2.4 GHz. v_exp_f32 issues at half the rate of
# a plain fp32 op on gfx950 (16 lanes per clock per SIMD unpacked); the
# probe (--exp-probe, and the `probe` object of every default line) measures
# what the chip sustains. One exponential per (i, j) pair and half-step.
EXP_PEAK_PER_S = 256 * 4 * 8 * 2.4e9

# HBM bytes of one launch of the dominant kernel, from rocprofv3 --pmc
# FETCH_SIZE / WRITE_SIZE runs (scaled by the copy-kernel calibration), valid
# only for the kernel source they were taken on.
TRAFFIC = {
    "c2": {"kernels_sha256": "8926fdd03eec55c0dffccb62985e1fa693923b4386f689ad302bc020c3d180aa",
           "splits": 16,
           "bytes_per_launch": 34082816,
           "source": "profiles/lse_pipe_kernel_c2_n20000_d64_f32half2_hbm_traffic.md"},
}
# Sources of the register-resident log-sum-exp kernels the counters describe.
KERNEL_SRCS = [os.path.join(ROOT, "streaming_sinkhorn_amd", "csrc", f)
               for f in ("kernels.hip", "device_common.h")]

METRIC = "Sinkhorn n*m*iters/sec + % MFMA/exp roofline at n=m=20k, d=64, eps=0.1"


# What the fp32 products of each operand mode run as (ot_solve_info.operand_mode).
DTYPE_LABEL = {0: "f32", 1: "bf16", 2: "f32 (3xbf16 split)", 3: "f32 (2xfp16 split)"}


def lse_roofline(pairs, d, dtype, mode, avg_s):
    """Roofline of one log-sum-exp launch over `pairs` (i, j) pairs at dimension d.

    Method work per launch: 2 d flops per pair on the matrix cores and one
    exponential per pair. The matrix work is priced at the peak of the unit
    the contraction runs on: fp16 for fp32 points in the default two-part fp16
    split (mode 3), bf16 for the three-part bf16 split (mode 2) and for bf16
    points (mode 1), fp32 for OT_NATIVE_F32 (mode 0). frac = the larger ideal
    time over the measured one. executed_frac prices what the kernel issues:
    3 (mode 3) or 6 (mode 2) products per fp32 product, plus nothing for the
    bias instruction."""
    unit = {3: "f16", 2: "bf16", 1: "bf16", 0: "f32"}[mode]
    peak = MFMA_PEAK_TFLOPS[unit]
    alg_flops = 2.0 * pairs * d
    executed = alg_flops * {3: 3.0, 2: 6.0}.get(mode, 1.0)
    t_mfma = alg_flops / (peak * 1e12)
    t_exp = pairs / EXP_PEAK_PER_S
    if t_mfma >= t_exp:
        roof = {"bound": "mfma", "achieved": alg_flops / avg_s / 1e12, "peak": peak,
                "unit": "TFLOP/s", "frac": t_mfma / avg_s}
    else:
        roof = {"bound": "alu", "achieved": pairs / avg_s / 1e9, "peak": EXP_PEAK_PER_S / 1e9,
                "unit": "Gexp/s", "frac": t_exp / avg_s}
    roof.update({
        "matrix_unit": unit,
        "method_flops_per_launch": alg_flops,
        "exps_per_launch": pairs,
        "ideal_us": {"mfma": t_mfma * 1e6, "exp": t_exp * 1e6},
        "executed_matrix_flops_per_launch": executed,
        "executed_frac": executed / (peak * 1e12) / avg_s,
    })
    return roof


def kernel_sha():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(workload, splits):
    """Counter-measured HBM bytes per launch, if taken on these kernel sources
    and this column-split count (it sets the partials written)."""
    rec = TRAFFIC.get(workload)
    if not rec or rec["kernels_sha256"] != kernel_sha() or rec["splits"] != splits:
        return None
    return rec["bytes_per_launch"]


# Inputs of the oracle sample, set before the worker pool forks (the workers
# read them copy-on-write).
_CPU_JOB = {}


def _oracle_chunk(task):
    """One block of the oracle sample in a worker: f half-step rows or g
    half-step columns [lo, hi)."""
    import oracle

    side, lo, hi = task
    j = _CPU_JOB
    if side == "f":
        oracle.update_f_rows(j["X"][lo:hi], j["Y"], j["g"], j["b"], j["eps"])
    else:
        oracle.update_g_cols(j["X"], j["Y"][lo:hi], j["f"], j["a"], j["eps"])
    return hi - lo


def _noop(_):
    return 0


def host_workers():
    """CPU threads for the oracle baseline: this process's CPUs, at most 16
    (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(data, budget=1.05e10):
    """fp64 oracle on a row sample of the same workload, one worker process per
    host CPU: one f half-step for `rows` rows of X and one g half-step for
    `rows` columns of Y, split into row blocks, reported in n*m*iterations/s.
    `budget` bounds pairs x d per worker (about 10 s of numpy each).

    Runs before the GPU is first used: the workers are forked from this
    process and only run numpy."""
    import multiprocessing

    import numpy as np

    w = data["w"]
    workers = host_workers()
    rows = int(max(8, min(w.n, w.m, budget * workers / (w.d * (w.n + w.m)))))
    _CPU_JOB.update(X=data["X"].astype(np.float64), Y=data["Y"].astype(np.float64),
                    a=data["a"].astype(np.float64), b=data["b"].astype(np.float64),
                    f=np.zeros(w.n), g=np.zeros(w.m), eps=w.eps)
    chunk = max(1, -(-rows // (2 * workers)))
    tasks = [(side, lo, min(rows, lo + chunk)) for side in ("f", "g") for lo in range(0, rows, chunk)]
    with multiprocessing.get_context("fork").Pool(workers) as pool:
        pool.map(_noop, range(workers))  # workers started before the clock
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_chunk, tasks, chunksize=1))
        dt = time.perf_counter() - t0
    _CPU_JOB.clear()
    assert done == 2 * rows
    pairs = rows * w.m + w.n * rows
    return {
        "value": pairs / 2.0 / dt,
        "unit": "n*m*iters/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle in {workers} worker processes (one per host CPU; host has "
                  f"{os.cpu_count()} CPUs): f half-step on {rows} rows x {w.m} columns and g "
                  f"half-step on {rows} columns x {w.n} rows of the same workload ({pairs} pairs, "
                  f"{dt:.1f} s); one iteration = two half-steps",
    }


def copy_probe(mib):
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "copies": 3}), flush=True)


def rate_probes(reps=3, all_kinds=False):
    """Throughput of the exponential and of the fp16 matrix instruction, each
    from the library's probe kernel timed with HIP events on its stream; with
    all_kinds also the fp16 matrix rate at two waves per SIMD with one and two
    accumulation chains per wave, and that of the d = 64 fp32 pass's per-stage
    instruction mix (include/flashot_probe.h)."""
    import torch

    import streaming_sinkhorn_amd as ssa

    out = {}
    kinds = [(ssa.OT_PROBE_EXP2, "exp2_per_s", 4096), (ssa.OT_PROBE_MFMA_F16, "mfma_f16_tflops", 1024)]
    if all_kinds:
        kinds += [(ssa.OT_PROBE_MFMA_F16_1C2W, "mfma_f16_1chain_2waves_tflops", 2048),
                  (ssa.OT_PROBE_MFMA_F16_2C2W, "mfma_f16_2chains_2waves_tflops", 1024),
                  (ssa.OT_PROBE_MIX_2W, "mix_2waves_mfma_f16_tflops", 128)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for kind, name, iters in kinds:
            ssa.ot_probe_rate(kind, iters)  # warm-up
            best = None
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                buf, work = ssa.ot_probe_rate(kind, iters)
                e1.record(stream)
                stream.synchronize()
                rate = work / (e0.elapsed_time(e1) / 1e3)
                best = rate if best is None else max(best, rate)
                del buf
            out[name] = best / 1e12 if name.endswith("tflops") else best
    out["note"] = ("best of 3 launches, 2048 workgroups of 256 threads; exp2: 8 independent "
                   "chains per lane; fp16 MFMA: 4 independent 32x32x16 chains per wave")
    return out


def gemm_probe():
    import torch

    torch.manual_seed(0)
    out = {}
    for m, k, n, reps in ((16384, 16384, 16384, 5), (20000, 1024, 20000, 10)):
        a = torch.randn(m, k, device="cuda:0", dtype=torch.bfloat16)
        b = torch.randn(k, n, device="cuda:0", dtype=torch.bfloat16)
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"bf16_{m}x{k}x{n}_tflops"] = 2.0 * m * n * k / ms / 1e9
        del a, b, c
    print(json.dumps(out), flush=True)


def hvp_cpu_baseline(data, tau, K, rows=3000):
    """fp64 oracle HVP (dense coupling, damped Schur CG) on the first `rows` points
    of each cloud; seconds per call, and that time scaled to the full n x m by
    the pair count."""
    import numpy as np

    import oracle

    w = data["w"]
    X = data["X"][:rows].astype(np.float64)
    Y = data["Y"][:rows].astype(np.float64)
    A = data["A"][:rows].astype(np.float64)
    a = np.full(rows, 1.0 / rows)
    b = np.full(rows, 1.0 / rows)
    f, g = oracle.sinkhorn(oracle.cost_matrix(X, Y), a, b, w.eps, 20)
    # the oracle's dense products run in numpy's BLAS: its thread count is the
    # number of host threads the sample used
    try:
        from threadpoolctl import threadpool_info
        cores = max([1] + [p.get("num_threads", 1) for p in threadpool_info()
                           if p.get("user_api") == "blas"])
    except Exception:  # threadpoolctl missing: numpy's BLAS thread count unknown
        cores = None
    t0 = time.perf_counter()
    oracle.hvp.hvp_schur_cg(X, Y, a, b, f, g, w.eps, A, tau=tau, iters=K)
    dt = time.perf_counter() - t0
    return {
        "value": dt * (float(w.n) * w.m) / (rows * rows),
        "unit": "s per HVP (scaled to the full n*m by pair count)",
        "cores": cores,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle HVP (dense coupling, K={K} CG iterations) on n=m={rows} "
                  f"points of the same workload: {dt:.2f} s; scaled by n*m / {rows}^2",
    }


def hvp_main(args):
    """Streaming Hessian-vector product on the page's HVP benchmark shape."""
    import torch

    import streaming_sinkhorn_amd as ssa
    import workloads

    ssa.lib()
    name = args.workload if args.workload.startswith("hvp") else "hvp_n50k_d64"
    data = workloads.make(name)
    w = data["w"]
    K, tau = args.hvp_iters, 1e-5
    dev = "cuda:0"
    torch.cuda.set_device(0)
    X = torch.from_numpy(data["X"]).to(dev)
    Y = torch.from_numpy(data["Y"]).to(dev)
    A = torch.from_numpy(data["A"]).to(dev)
    prob = ssa.problem(X, Y, w.eps)
    f = torch.zeros(w.n, device=dev)
    g = torch.zeros(w.m, device=dev)
    out = torch.empty((w.n, w.d), device=dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        ssa.ot_solve(prob, f, g, w.iters, want_info=False)  # potentials, outside the timed region
        ws = ssa.hvp_workspace(prob)
        for _ in range(args.warmup):
            ssa.ot_hvp(prob, f, g, A, tau=tau, max_iters=K, out=out, want_info=False, ws=ws)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for k in range(args.steps):
            ssa.ot_hvp(prob, f, g, A, tau=tau, max_iters=K, out=out, want_info=False, ws=ws)
            print(f"# hvp {k + 1}/{args.steps} enqueued", file=sys.stderr, flush=True)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    sec = (t1 - t0) / args.steps
    ev_sec = e0.elapsed_time(e1) / 1e3 / args.steps
    pairs = float(w.n) * w.m
    # Method work of one HVP, pass by pass, each contraction against the peak
    # of the unit it runs on and one exponential per pair; the ideal time of a
    # pass is the larger of its matrix and exponential times, and the HVP's is
    # their sum (frac = ideal / measured):
    # - 2 K + 2 transport-vector passes (conjugate gradients and the marginals
    #   they use): 2 d flops per pair on the fp16 matrix cores (fp32 points as
    #   the two-part fp16 split); the value sum is vector work;
    # - 3 transport-matrix passes with d, d + 2 and d + 1 value columns: scores
    #   on the fp32 matrix instruction (2 d per pair), values on the fp16
    #   matrix cores (2 per pair and column);
    # - the Hadamard-weighted pass: two score tiles and the values, all fp32
    #   (4 d + 2 d per pair).
    f16 = MFMA_PEAK_TFLOPS["f16"] * 1e12
    f32 = MFMA_PEAK_TFLOPS["f32"] * 1e12
    t_exp = pairs / EXP_PEAK_PER_S
    vec = (2 * K + 2) * max(pairs * 2.0 * w.d / f16, t_exp)
    mat = sum(max(pairs * 2.0 * w.d / f32 + pairs * 2.0 * cols / f16, t_exp)
              for cols in (w.d, w.d + 2, w.d + 1))
    had = max(pairs * 6.0 * w.d / f32, t_exp)
    ideal = vec + mat + had
    res = {
        "metric": f"streaming HVP time per call (n=m={w.n}, d={w.d}, K={K} CG, tau={tau})",
        "value": sec,
        "unit": "s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (2xfp16 split scores; fp32 transport-matrix scores)",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: n={w.n}, m={w.m}, d={w.d}, fp32 points uniform in "
                               f"[0,1]^d, uniform weights, eps={w.eps}; potentials from {w.iters} "
                               f"iterations (untimed); HVP with K={K} fixed CG iterations, tau={tau}",
                   "n": w.n, "m": w.m, "d": w.d, "eps": w.eps, "cg_iters": K,
                   "transport_passes": 2 * K + 4},
        "roofline": {"bound": "mfma", "achieved": ideal / ev_sec * MFMA_PEAK_TFLOPS["f16"],
                     "peak": MFMA_PEAK_TFLOPS["f16"],
                     "unit": "TFLOP/s (fp16-equivalent)", "frac": ideal / ev_sec,
                     "traffic": None,
                     "kernel": "all streamed passes of one HVP (vector passes: lse_*_kernel with a "
                               "value column; matrix passes: apply_*_kernel); the method's work of "
                               "each pass against the peak of the unit it runs on (fp32 work "
                               "weighted by the fp16/fp32 peak ratio), over the event-timed call",
                     "ideal_sec": ideal, "event_sec_per_hvp": ev_sec},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = hvp_cpu_baseline(data, tau, K)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--iters", type=int, default=None)
    ap.add_argument("--splits", type=int, default=0,
                    help="column splits of both half-steps (0: the library's choice)")
    ap.add_argument("--splits-f", type=int, default=None, help="column splits of the f half-step")
    ap.add_argument("--splits-g", type=int, default=None, help="column splits of the g half-step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--gemm-probe", action="store_true")
    ap.add_argument("--exp-probe", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps with the iterations replayed from HIP graphs (the "
                         "roofline's per-launch times then come from one extra plain step)")
    ap.add_argument("--schedule", default="alternating", choices=["alternating", "symmetric"])
    ap.add_argument("--native-f32", action="store_true",
                    help="form fp32 scores with the fp32 matrix instruction instead of the "
                         "two-part fp16 split")
    ap.add_argument("--split-bf16", action="store_true",
                    help="form fp32 scores from three bf16 parts per value (six products)")
    ap.add_argument("--hvp", action="store_true",
                    help="time the streaming Hessian-vector product instead of the solve")
    ap.add_argument("--hvp-iters", type=int, default=50, help="CG iterations K of --hvp")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path runs "
              f"on a single MI355X and multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)
    if args.gemm_probe:
        gemm_probe()
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.exp_probe:
        import streaming_sinkhorn_amd as ssa

        ssa.lib()
        res = rate_probes(all_kinds=True)
        res["exp2_peak_per_s"] = EXP_PEAK_PER_S
        res["mfma_f16_peak_tflops"] = MFMA_PEAK_TFLOPS["f16"]
        print(json.dumps(res), flush=True)
        return
    if args.hvp:
        hvp_main(args)
        return

    import torch

    import streaming_sinkhorn_amd as ssa
    import workloads

    if not os.path.exists(ssa.LIB_PATH):
        ssa.lib()  # raises: fail loudly before any work if the HIP library is missing
    data = workloads.make(args.workload)
    w = data["w"]
    # The oracle baseline runs first, in worker processes forked before this
    # process touches the GPU.
    cpu = None if args.no_cpu_baseline else cpu_baseline(data)
    ssa.lib()
    T = args.iters or w.iters
    sf = args.splits if args.splits_f is None else args.splits_f
    sg = args.splits if args.splits_g is None else args.splits_g
    dev = "cuda:0"
    torch.cuda.set_device(0)

    def to_dev(arr):
        t = torch.from_numpy(arr).to(dev)
        return t.to(torch.bfloat16) if w.dtype == "bf16" else t

    X, Y = to_dev(data["X"]), to_dev(data["Y"])
    a = torch.from_numpy(data["a"]).to(dev)
    b = torch.from_numpy(data["b"]).to(dev)
    V = to_dev(data["V"]) if w.v_cols else None
    U = to_dev(data["U"]) if w.u_cols else None
    xs = torch.empty(w.n, device=dev)
    ys = torch.empty(w.m, device=dev)
    prob = ssa.problem(X, Y, w.eps, a, b, x_sqn=xs, y_sqn=ys, native_f32=args.native_f32,
                       split_bf16=args.split_bf16)
    f = torch.zeros(w.n, device=dev)
    g = torch.zeros(w.m, device=dev)
    r = torch.empty(w.n, device=dev)
    c = torch.empty(w.m, device=dev)
    out_grad = torch.empty((w.n, w.d), device=dev) if w.grad else None
    out_pv = torch.empty((w.n, w.v_cols), device=dev) if w.v_cols else None
    out_ptu = torch.empty((w.m, w.u_cols), device=dev) if w.u_cols else None
    stream = torch.cuda.Stream()
    infos = []
    ws = {}

    def step(record, timing=True):
        ssa.ot_sqnorms(X, xs)
        ssa.ot_sqnorms(Y, ys)
        info = ssa.ot_solve(prob, f, g, T, splits_f=sf, splits_g=sg,
                            timing=timing, ws=ws.get("solve"), schedule=args.schedule)
        if w.grad:
            ssa.ot_apply_plan(prob, f, g, flags=ssa.OT_GRAD, out=out_grad, marg=r, ws=ws.get("grad"))
        if w.v_cols:
            ssa.ot_apply_plan(prob, f, g, V, out=out_pv, marg=r, ws=ws.get("pv"))
        if w.u_cols:
            ssa.ot_apply_plan(prob, f, g, U, flags=ssa.OT_TRANSPOSE, out=out_ptu, marg=c,
                              ws=ws.get("ptu"))
        if record:
            infos.append(info)

    with torch.cuda.stream(stream):
        # Workspaces sized and allocated once, outside the timed region.
        ws["solve"] = ssa.solve_workspace(prob, T, splits_f=sf, splits_g=sg)
        if w.grad:
            ws["grad"] = ssa.apply_workspace(prob, flags=ssa.OT_GRAD)
        if w.v_cols:
            ws["pv"] = ssa.apply_workspace(prob, V)
        if w.u_cols:
            ws["ptu"] = ssa.apply_workspace(prob, U, flags=ssa.OT_TRANSPOSE)
        for _ in range(args.warmup):
            step(False, not args.graph)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(not args.graph, not args.graph)
            print(f"# step {k + 1}/{args.steps} done", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if args.graph:
            # per-launch events need plain launches: one more step, after the timed ones
            step(True)
            torch.cuda.synchronize()
        else:
            # the same steps with the iterations replayed from HIP graphs (how
            # ot_solve runs by default), timed separately, for reference
            for _ in range(args.warmup):
                step(False, False)
            torch.cuda.synchronize()
            g0 = time.perf_counter()
            for _ in range(args.steps):
                step(False, False)
            torch.cuda.synchronize()
            g1 = time.perf_counter()
            graph_replay = {"value": w.n * w.m * T / ((g1 - g0) / args.steps),
                            "ms_per_step": (g1 - g0) * 1e3 / args.steps,
                            "note": "same steps, iterations replayed from HIP graphs (16 per "
                                    "graph), timed after the event-timed steps"}

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = w.n * w.m * T / ((t1 - t0) / args.steps)
    lse_ms = sum(i["lse_ms"] for i in infos)
    lse_n = sum(i["lse_launches"] for i in infos)
    avg_lse_s = lse_ms / lse_n / 1e3
    pairs = float(w.n) * w.m
    mode = infos[-1]["operand_mode"]
    roof = lse_roofline(pairs, w.d, w.dtype, mode, avg_lse_s)
    roof["traffic"] = traffic_for(args.workload, infos[-1]["splits_f"])
    roof.update({"kernel": "streamed log-sum-exp pass (lse_*_kernel)",
                 "avg_launch_us": avg_lse_s * 1e6, "launches": lse_n})
    last = infos[-1]
    outputs = ["f", "g", "marginal errors"]
    if w.grad:
        outputs.append("P*Y gradient")
    if w.v_cols:
        outputs.append(f"P*V (V m x {w.v_cols})")
    if w.u_cols:
        outputs.append(f"P^T*U (U n x {w.u_cols})")
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "n*m*iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_LABEL[mode] if w.dtype == "f32" else w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: n={w.n}, m={w.m}, d={w.d}, {w.dtype} points, eps={w.eps}, {T} "
                        f"{args.schedule} iterations from zero potentials; outputs: {', '.join(outputs)}",
            "n": w.n, "m": w.m, "d": w.d, "eps": w.eps, "iters": T,
            "splits_f": last["splits_f"], "splits_g": last["splits_g"],
            "launch_mode": ("HIP graph replay (roofline from one extra plain step)" if args.graph
                         else "plain launches with HIP events"),
            "operand_mode": ["fp32 MFMA", "bf16 MFMA", "fp32 as 3-part bf16 split on bf16 MFMA",
                             "fp32 as 2-part fp16 split on fp16 MFMA"][last["operand_mode"]],
        },
        "roofline": roof,
        "marg_err_row": last["marg_err_row"],
        "marg_err_col": last["marg_err_col"],
        **({} if args.graph else {"graph_replay": graph_replay}),
    }
    with torch.cuda.stream(stream):
        out["probe"] = rate_probes()
        if pairs <= 4.0e8:
            out["iteration_graph_us"] = iteration_latency(
                ssa, prob, f, g, ws["solve"], stream,
                dict(splits_f=sf, splits_g=sg, schedule=args.schedule))
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def iteration_latency(ssa, prob, f, g, ws, stream, opts, short=20, long=60, reps=3):
    """Time of one iteration with graph replay, without the per-call work
    (norms, operand packing, final marginal errors): the difference of a
    `long`- and a `short`-iteration ot_solve (best of `reps` each, HIP events
    on the stream), divided by long - short. After the timed steps; not part
    of `value`."""
    import torch

    best = {}
    for T in (short, long):
        ssa.ot_solve(prob, f, g, T, want_info=False, ws=ws, **opts)  # graph capture for this count
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ssa.ot_solve(prob, f, g, T, want_info=False, ws=ws, **opts)
            e1.record(stream)
            stream.synchronize()
            times.append(e0.elapsed_time(e1))
        best[T] = min(times)
    return (best[long] - best[short]) * 1e3 / (long - short)


if __name__ == "__main__":
    main()
