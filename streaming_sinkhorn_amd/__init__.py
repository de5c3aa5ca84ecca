"""Python binding of ``libflashot.so``: streamed log-domain Sinkhorn on MI355X.

Argument marshalling only. Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/flashot.h``; this module turns
torch tensors into device pointers, allocates the caller-owned workspace with
torch, passes torch's current stream, and maps status codes to exceptions.
There is no CPU fallback: if the library is not built every entry point raises.

Functions (same names as the C entry points):
    ot_sqnorms(pts, out=None)
    ot_update_f(prob, g, f, err=None)
    ot_update_g(prob, f, g, err=None)
    ot_solve(prob, f, g, iters, ...)
    ot_apply_plan(prob, f, g, V=None, flags=0, out=None, marg=None)
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflashot.so")
INCLUDE_DIR = os.path.join(os.path.dirname(HERE), "include")
HEADER_PATH = os.path.join(INCLUDE_DIR, "flashot.h")

OT_OK, OT_ERR_INVALID_ARG, OT_ERR_UNSUPPORTED, OT_ERR_WORKSPACE, OT_ERR_HIP, OT_ERR_NONFINITE = range(6)
OT_F32, OT_BF16 = 0, 1
OT_INIT_ZERO, OT_INIT_GIVEN = 0, 1
OT_TRANSPOSE, OT_GRAD, OT_BARY = 1, 2, 4
OT_NATIVE_F32 = 1
OT_COST_AFFINE = 2
OT_SPLIT_BF16 = 4
OT_SCHED_ALTERNATING, OT_SCHED_SYMMETRIC = 0, 1
OT_PROBE_EXP2, OT_PROBE_MFMA_F16, OT_PROBE_MFMA_F16_1C2W, OT_PROBE_MFMA_F16_2C2W, OT_PROBE_MIX_2W = range(5)
_SCHEDULES = {"alternating": OT_SCHED_ALTERNATING, "symmetric": OT_SCHED_SYMMETRIC}


class OtError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where} failed with status {code}: {msg}")
        self.code = code


class OtProblem(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("n", ctypes.c_int64), ("m", ctypes.c_int64), ("d", ctypes.c_int64),
        ("ldx", ctypes.c_int64), ("ldy", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("eps", ctypes.c_float),
        ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
        ("x_sqn", ctypes.c_void_p), ("y_sqn", ctypes.c_void_p),
        ("flags", ctypes.c_int32),
    ]


class OtSolveOpts(ctypes.Structure):
    _fields_ = [
        ("iters", ctypes.c_int32), ("tol", ctypes.c_float), ("check_every", ctypes.c_int32),
        ("init", ctypes.c_int32), ("use_graph", ctypes.c_int32),
        ("splits_f", ctypes.c_int32), ("splits_g", ctypes.c_int32), ("timing", ctypes.c_int32),
        ("schedule", ctypes.c_int32), ("eps_start", ctypes.c_float), ("eps_decay", ctypes.c_float),
    ]


class OtSolveInfo(ctypes.Structure):
    _fields_ = [
        ("iters_done", ctypes.c_int32), ("nonfinite", ctypes.c_int32),
        ("marg_err_row", ctypes.c_float), ("marg_err_col", ctypes.c_float),
        ("lse_ms", ctypes.c_float), ("lse_launches", ctypes.c_int32),
        ("splits_f", ctypes.c_int32), ("splits_g", ctypes.c_int32),
        ("operand_mode", ctypes.c_int32),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class OtHvpOpts(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("max_iters", ctypes.c_int32), ("tol", ctypes.c_float)]


class OtHvpInfo(ctypes.Structure):
    _fields_ = [("cg_iters", ctypes.c_int32), ("breakdown", ctypes.c_int32),
                ("cg_rel_residual", ctypes.c_float)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """Load libflashot.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m streaming_sinkhorn_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    szp = ctypes.POINTER(ctypes.c_size_t)
    pp = ctypes.POINTER(OtProblem)
    L.ot_sqnorms.argtypes = [vp, i32, i64, i64, i64, vp, vp]
    L.ot_update_f.argtypes = [pp, vp, vp, vp, vp, szp, vp]
    L.ot_update_g.argtypes = [pp, vp, vp, vp, vp, szp, vp]
    L.ot_solve.argtypes = [pp, vp, vp, ctypes.POINTER(OtSolveOpts), ctypes.POINTER(OtSolveInfo), vp, szp, vp]
    L.ot_apply_plan.argtypes = [pp, vp, vp, vp, i32, i64, i64, i32, vp, vp, vp, szp, vp]
    L.ot_sinkhorn_divergence.argtypes = [pp, ctypes.POINTER(OtSolveOpts), vp, vp, vp, vp, vp, vp,
                                         szp, vp]
    L.ot_prep_cosine.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    L.ot_prep_labels.argtypes = [vp, i32, i64, i64, i64, vp, vp, i32, i32, vp, vp, vp]
    L.ot_apply_hadamard.argtypes = [pp, vp, vp, vp, i64, vp, i64, i64, vp, vp, szp, vp]
    L.ot_hvp.argtypes = [pp, vp, vp, vp, i64, ctypes.POINTER(OtHvpOpts), vp,
                         ctypes.POINTER(OtHvpInfo), vp, szp, vp]
    L.ot_probe_rate.argtypes = [i32, i64, ctypes.c_int32, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.ot_solve_static.argtypes = [pp, vp, vp, ctypes.POINTER(OtSolveOpts), ctypes.POINTER(OtSolveInfo), vp]
    L.ot_solve_static.restype = ctypes.c_int
    L.ot_static_scratch_bytes.argtypes = []
    L.ot_static_scratch_bytes.restype = ctypes.c_size_t
    for fn in ("ot_sqnorms", "ot_update_f", "ot_update_g", "ot_solve", "ot_apply_plan",
               "ot_apply_hadamard", "ot_hvp", "ot_prep_cosine", "ot_prep_labels",
               "ot_sinkhorn_divergence", "ot_probe_rate"):
        getattr(L, fn).restype = ctypes.c_int
    L.ot_last_error.restype = ctypes.c_char_p
    L.ot_last_error.argtypes = []
    L.ot_version.restype = ctypes.c_char_p
    L.ot_version.argtypes = []
    _lib = L
    return L


def header_entry_points() -> list[str]:
    """Names of the functions declared in the headers under include/."""
    names = []
    for fn in sorted(os.listdir(INCLUDE_DIR)):
        if fn.endswith(".h"):
            txt = open(os.path.join(INCLUDE_DIR, fn)).read()
            names += re.findall(r"^\s*(?:int|size_t|const char\*)\s+(ot_\w+)\s*\(", txt, re.M)
    return names


def _check(code: int, where: str):
    if code != OT_OK:
        msg = lib().ot_last_error().decode(errors="replace")
        raise OtError(code, where, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return OT_F32
    if t.dtype == torch.bfloat16:
        return OT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _rows(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride along dimension 1")
    return t.shape[0], t.shape[1], t.stride(0)


def _vec(t, name, length, device):
    if t is None:
        return None
    if t.dtype != torch.float32 or t.dim() != 1 or t.numel() != length or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 vector of length {length}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    return t


@dataclass
class Problem:
    """Keeps the tensors of an ot_problem alive next to its C struct."""
    X: torch.Tensor
    Y: torch.Tensor
    eps: float
    a: torch.Tensor | None = None
    b: torch.Tensor | None = None
    x_sqn: torch.Tensor | None = None
    y_sqn: torch.Tensor | None = None
    native_f32: bool = False
    affine: bool = False
    split_bf16: bool = False

    def __post_init__(self):
        n, d, ldx = _rows(self.X, "X")
        m, d2, ldy = _rows(self.Y, "Y")
        if d != d2:
            raise ValueError("X and Y must have the same number of columns")
        if self.X.dtype != self.Y.dtype:
            raise ValueError("X and Y must have the same dtype")
        dev = self.X.device
        self.device = dev
        self.n, self.m, self.d = n, m, d
        self.c = OtProblem(
            _ptr(self.X), _ptr(self.Y), n, m, d, ldx, ldy, _dtype_code(self.X), float(self.eps),
            _ptr(_vec(self.a, "a", n, dev)), _ptr(_vec(self.b, "b", m, dev)),
            _ptr(_vec(self.x_sqn, "x_sqn", n, dev)), _ptr(_vec(self.y_sqn, "y_sqn", m, dev)),
            (OT_NATIVE_F32 if self.native_f32 else 0) | (OT_COST_AFFINE if self.affine else 0)
            | (OT_SPLIT_BF16 if self.split_bf16 else 0))


def problem(X, Y, eps, a=None, b=None, x_sqn=None, y_sqn=None, native_f32=False,
            affine=False, split_bf16=False) -> Problem:
    """fp32 points form their scores from two fp16 parts per value by default;
    native_f32 uses fp32 MFMA and split_bf16 three bf16 parts instead.
    affine: cost alpha_i + beta_j - <x_i, y_j> with alpha = x_sqn, beta = y_sqn (required)."""
    return Problem(X, Y, eps, a, b, x_sqn, y_sqn, native_f32, affine, split_bf16)


def _workspace(query, ws, device):
    size = ctypes.c_size_t(0)
    _check(query(None, ctypes.byref(size)), "workspace query")
    need = size.value
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    elif ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")
    size.value = ws.numel()
    return ws, size


def ot_sqnorms(pts: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    rows, d, ld = _rows(pts, "pts")
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=pts.device)
    _check(lib().ot_sqnorms(_ptr(pts), _dtype_code(pts), rows, d, ld, _ptr(out), _stream(pts.device)),
           "ot_sqnorms")
    return out


def _update(fn, name, prob, src, dst, err, ws):
    L = lib()
    c_fn = getattr(L, fn)
    st = _stream(prob.device)
    pp = ctypes.byref(prob.c)
    ws, size = _workspace(lambda w, s: c_fn(pp, _ptr(src), _ptr(dst), _ptr(err), w, s, st), ws, prob.device)
    _check(c_fn(pp, _ptr(src), _ptr(dst), _ptr(err), _ptr(ws), ctypes.byref(size), st), name)
    return dst


def ot_update_f(prob: Problem, g, f, err=None, ws=None):
    """One f half-step from g, written into f (in place); optional device scalar err."""
    return _update("ot_update_f", "ot_update_f", prob, g, f, err, ws)


def ot_update_g(prob: Problem, f, g, err=None, ws=None):
    """One g half-step from f, written into g (in place); optional device scalar err."""
    return _update("ot_update_g", "ot_update_g", prob, f, g, err, ws)


def _solve_opts(iters, tol=0.0, check_every=1, init_given=False, use_graph=True, splits_f=0,
                splits_g=0, timing=False, schedule="alternating", eps_start=0.0, eps_decay=0.5):
    return OtSolveOpts(int(iters), float(tol), int(check_every),
                       OT_INIT_GIVEN if init_given else OT_INIT_ZERO, int(bool(use_graph)),
                       int(splits_f), int(splits_g), int(bool(timing)), _SCHEDULES[schedule],
                       float(eps_start), float(eps_decay))


def ot_solve_static(prob: Problem, f, g, iters: int, tol: float = 0.0, check_every: int = 1,
                    init_given: bool = False, want_info: bool = True, schedule: str = "alternating",
                    eps_start: float = 0.0, eps_decay: float = 0.5):
    """ot_solve on the library's static device scratch (no workspace, no allocation,
    plain launches). Returns the info dict (None if want_info is False)."""
    L = lib()
    opts = _solve_opts(iters, tol, check_every, init_given, False, 0, 0, False, schedule,
                       eps_start, eps_decay)
    info = OtSolveInfo()
    pinfo = ctypes.byref(info) if want_info else None
    _check(L.ot_solve_static(ctypes.byref(prob.c), _ptr(f), _ptr(g), ctypes.byref(opts), pinfo,
                             _stream(prob.device)), "ot_solve_static")
    return info.as_dict() if want_info else None


def static_scratch_bytes() -> int:
    return int(lib().ot_static_scratch_bytes())


def ot_sinkhorn_divergence(prob: Problem, iters: int, f=None, g=None, schedule: str = "alternating",
                           eps_start: float = 0.0, eps_decay: float = 0.5, ws=None):
    """Debiased Sinkhorn divergence. Returns (values, f, g, f_xx, g_yy) with values a
    host tuple (S, OT(mu, nu), OT(mu, mu), OT(nu, nu)); the call synchronises."""
    L = lib()
    dev = prob.device
    f = torch.zeros(prob.n, device=dev) if f is None else f
    g = torch.zeros(prob.m, device=dev) if g is None else g
    fxx = torch.empty(prob.n, device=dev)
    gyy = torch.empty(prob.m, device=dev)
    out = torch.empty(4, device=dev)
    opts = _solve_opts(iters, schedule=schedule, eps_start=eps_start, eps_decay=eps_decay)
    st = _stream(dev)
    pp = ctypes.byref(prob.c)
    args = lambda w, s: L.ot_sinkhorn_divergence(pp, ctypes.byref(opts), _ptr(f), _ptr(g), _ptr(fxx),
                                                 _ptr(gyy), _ptr(out), w, s, st)
    ws, size = _workspace(args, ws, dev)
    _check(args(_ptr(ws), ctypes.byref(size)), "ot_sinkhorn_divergence")
    vals = tuple(float(v) for v in out.cpu())
    return vals, f, g, fxx, gyy


def ot_solve(prob: Problem, f, g, iters: int, tol: float = 0.0, check_every: int = 1,
             init_given: bool = False, use_graph: bool = True, splits_f: int = 0,
             splits_g: int = 0, timing: bool = False, want_info: bool = True, ws=None,
             schedule: str = "alternating", eps_start: float = 0.0, eps_decay: float = 0.5):
    """Sinkhorn iterations into f, g (schedule "alternating" or "symmetric"; eps-scaling
    from eps_start by eps_decay per iteration when eps_start > eps).
    Returns the info dict (None if want_info is False)."""
    L = lib()
    opts = _solve_opts(iters, tol, check_every, init_given, use_graph, splits_f, splits_g, timing,
                       schedule, eps_start, eps_decay)
    info = OtSolveInfo()
    pinfo = ctypes.byref(info) if want_info else None
    st = _stream(prob.device)
    pp = ctypes.byref(prob.c)
    ws, size = _workspace(lambda w, s: L.ot_solve(pp, _ptr(f), _ptr(g), ctypes.byref(opts), pinfo, w, s, st),
                          ws, prob.device)
    _check(L.ot_solve(pp, _ptr(f), _ptr(g), ctypes.byref(opts), pinfo, _ptr(ws), ctypes.byref(size), st),
           "ot_solve")
    return info.as_dict() if want_info else None


def ot_apply_plan(prob: Problem, f, g, V=None, flags: int = 0, out=None, marg=None, ws=None):
    """out = P V (P^T U with OT_TRANSPOSE; barycentric with OT_BARY; X-gradient with OT_GRAD)."""
    L = lib()
    tr = bool(flags & OT_TRANSPOSE)
    rows = prob.m if tr else prob.n
    if flags & OT_GRAD:
        vptr, vdt, cols, ldv = None, 0, prob.d, 0
    else:
        if V is None:
            raise ValueError("V is required unless OT_GRAD is set")
        vrows, cols, ldv = _rows(V, "V")
        if vrows != (prob.n if tr else prob.m):
            raise ValueError("V has the wrong number of rows")
        vptr, vdt = _ptr(V), _dtype_code(V)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=prob.device)
    st = _stream(prob.device)
    pp = ctypes.byref(prob.c)
    args = lambda w, s: L.ot_apply_plan(pp, _ptr(f), _ptr(g), vptr, vdt, cols, ldv, int(flags),
                                        _ptr(out), _ptr(marg), w, s, st)
    ws, size = _workspace(args, ws, prob.device)
    _check(args(_ptr(ws), ctypes.byref(size)), "ot_apply_plan")
    return out


def ot_prep_cosine(pts: torch.Tensor):
    """Cosine-cost features: (rows normalised to unit length, fp32; alpha = 1/2 per row).
    Use both clouds' outputs with problem(..., affine=True)."""
    rows, d, ld = _rows(pts, "pts")
    out = torch.empty((rows, d), dtype=torch.float32, device=pts.device)
    half = torch.empty(rows, dtype=torch.float32, device=pts.device)
    _check(lib().ot_prep_cosine(_ptr(pts), _dtype_code(pts), rows, d, ld, _ptr(out), _ptr(half),
                                _stream(pts.device)), "ot_prep_cosine")
    return out, half


def ot_prep_labels(pts: torch.Tensor, labels: torch.Tensor, W: torch.Tensor, side: int):
    """Label-augmented cost features (side 0: source [2x, -W[l, :]], side 1: target
    [y, one-hot(l)]) and the squared norms; use with problem(..., affine=True)."""
    rows, d, ld = _rows(pts, "pts")
    L = W.shape[0]
    if labels.dtype != torch.int32 or labels.numel() != rows or not labels.is_contiguous():
        raise ValueError("labels must be a contiguous int32 vector with one entry per row")
    if W.dtype != torch.float32 or W.shape != (L, L) or not W.is_contiguous():
        raise ValueError("W must be a contiguous float32 square matrix")
    out = torch.empty((rows, d + L), dtype=torch.float32, device=pts.device)
    sqn = torch.empty(rows, dtype=torch.float32, device=pts.device)
    _check(lib().ot_prep_labels(_ptr(pts), _dtype_code(pts), rows, d, ld, _ptr(labels), _ptr(W), L,
                                int(side), _ptr(out), _ptr(sqn), _stream(pts.device)),
           "ot_prep_labels")
    return out, sqn


def _f32_rows(t, name, rows, cols, device):
    r, c, ld = _rows(t, name)
    if t.dtype != torch.float32 or r != rows or c != cols or t.device != device:
        raise ValueError(f"{name} must be float32 of shape ({rows}, {cols}) on {device}")
    return ld


def ot_apply_hadamard(prob: Problem, f, g, A, V, out=None, ws=None):
    """out = (P . (A Y^T)) V, streamed from the potentials (fp32 points)."""
    L = lib()
    lda = _f32_rows(A, "A", prob.n, prob.d, prob.device)
    vrows, cols, ldv = _rows(V, "V")
    _f32_rows(V, "V", prob.m, cols, prob.device)
    if out is None:
        out = torch.empty((prob.n, cols), dtype=torch.float32, device=prob.device)
    st = _stream(prob.device)
    pp = ctypes.byref(prob.c)
    args = lambda w, s: L.ot_apply_hadamard(pp, _ptr(f), _ptr(g), _ptr(A), lda, _ptr(V), cols, ldv,
                                            _ptr(out), w, s, st)
    ws, size = _workspace(args, ws, prob.device)
    _check(args(_ptr(ws), ctypes.byref(size)), "ot_apply_hadamard")
    return out


def ot_hvp(prob: Problem, f, g, A, tau: float = 1e-5, max_iters: int = 50, tol: float = 0.0,
           out=None, want_info: bool = True, ws=None):
    """Hessian-vector product T A of OT_eps in X (damped Schur complement solved by
    conjugate gradients). Returns (out, info dict or None)."""
    L = lib()
    lda = _f32_rows(A, "A", prob.n, prob.d, prob.device)
    if out is None:
        out = torch.empty((prob.n, prob.d), dtype=torch.float32, device=prob.device)
    opts = OtHvpOpts(float(tau), int(max_iters), float(tol))
    info = OtHvpInfo()
    pinfo = ctypes.byref(info) if want_info else None
    st = _stream(prob.device)
    pp = ctypes.byref(prob.c)
    args = lambda w, s: L.ot_hvp(pp, _ptr(f), _ptr(g), _ptr(A), lda, ctypes.byref(opts), _ptr(out),
                                 pinfo, w, s, st)
    ws, size = _workspace(args, ws, prob.device)
    _check(args(_ptr(ws), ctypes.byref(size)), "ot_hvp")
    return out, (info.as_dict() if want_info else None)


def hvp_workspace(prob: Problem) -> torch.Tensor:
    """Allocate the workspace ot_hvp needs for this problem."""
    L = lib()
    opts = OtHvpOpts(0.0, 0, 0.0)
    size = ctypes.c_size_t(0)
    _check(L.ot_hvp(ctypes.byref(prob.c), None, None, None, prob.d, ctypes.byref(opts), None, None,
                    None, ctypes.byref(size), None), "ot_hvp workspace query")
    return torch.empty(max(size.value, 256), dtype=torch.uint8, device=prob.device)


def solve_workspace(prob: Problem, iters: int, splits_f: int = 0, splits_g: int = 0) -> torch.Tensor:
    """Allocate the workspace ot_solve needs for this problem (size query + torch allocation)."""
    L = lib()
    opts = OtSolveOpts(int(iters), 0.0, 1, OT_INIT_ZERO, 1, int(splits_f), int(splits_g), 0)
    size = ctypes.c_size_t(0)
    _check(L.ot_solve(ctypes.byref(prob.c), None, None, ctypes.byref(opts), None, None,
                      ctypes.byref(size), None), "ot_solve workspace query")
    return torch.empty(max(size.value, 256), dtype=torch.uint8, device=prob.device)


def apply_workspace(prob: Problem, V=None, flags: int = 0) -> torch.Tensor:
    """Allocate the workspace ot_apply_plan needs for this problem and value matrix."""
    L = lib()
    if flags & OT_GRAD:
        vdt, cols, ldv = 0, prob.d, prob.d
    else:
        _, cols, ldv = _rows(V, "V")
        vdt = _dtype_code(V)
    size = ctypes.c_size_t(0)
    _check(L.ot_apply_plan(ctypes.byref(prob.c), None, None, None, vdt, cols, ldv, int(flags),
                           None, None, None, ctypes.byref(size), None), "ot_apply_plan workspace query")
    return torch.empty(max(size.value, 256), dtype=torch.uint8, device=prob.device)


def ot_probe_rate(kind: int, iters: int, blocks: int = 2048):
    """Enqueue one throughput probe (an OT_PROBE_* kind) on the current stream.
    Returns (output tensor, work of the launch: exponentials or flops); the
    caller times the launch."""
    out = torch.empty(int(blocks) * 256, dtype=torch.float32, device="cuda")
    work = ctypes.c_double(0.0)
    _check(lib().ot_probe_rate(int(kind), int(iters), int(blocks), _ptr(out), ctypes.byref(work),
                               _stream(out.device)), "ot_probe_rate")
    return out, work.value


def version() -> str:
    return lib().ot_version().decode()
