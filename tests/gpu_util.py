"""Helpers shared by the GPU parity tests: move seeded inputs to the device and
call the HIP path through the binding. No arithmetic of the method lives here."""

from __future__ import annotations

import sys

import numpy as np
import torch

import streaming_sinkhorn_amd as ssa

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(arr, dtype="f32"):
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host64(t):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


# fp32 operand modes of the log-sum-exp passes: the default two-part fp16
# split, the three-part bf16 split, the fp32 matrix instruction
F32_MODES = ("half2", "split_bf16", "native")


def make_problem(data, eps=None, dtype=None, weights=True, native_f32=False, mode="half2"):
    w = data["w"]
    dtype = dtype or w.dtype
    X = dev(data["X"], dtype)
    Y = dev(data["Y"], dtype)
    a = dev(data["a"]) if weights else None
    b = dev(data["b"]) if weights else None
    prob = ssa.problem(X, Y, float(w.eps if eps is None else eps), a, b,
                       native_f32=native_f32 or mode == "native", split_bf16=mode == "split_bf16")
    return prob


def oracle_inputs(prob):
    """Exactly the values the GPU received, widened to float64."""
    X = host64(prob.X)
    Y = host64(prob.Y)
    a = host64(prob.a) if prob.a is not None else np.full(prob.n, np.float64(np.float32(1.0 / prob.n)))
    b = host64(prob.b) if prob.b is not None else np.full(prob.m, np.float64(np.float32(1.0 / prob.m)))
    return X, Y, a, b


def zeros(n):
    return torch.zeros(n, dtype=torch.float32, device=DEV)
