"""Builds libflashot.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m streaming_sinkhorn_amd.build   (or call build()).
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libflashot.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay disabled in all device code of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Streamed kernels only (kernels*.hip, apply_kernels.hip): MFMA results in ordinary VGPRs (the LSE
# reads them with the VALU right away) and no NaN canonicalisation around
# fmaxf. The auxiliary kernels keep full NaN semantics.
KERNEL_FLAGS = ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]

SOURCES = [
    ("kernels.hip", KERNEL_FLAGS),
    ("kernels_wide.hip", KERNEL_FLAGS),
    ("apply_kernels.hip", KERNEL_FLAGS),
    ("aux_kernels.hip", []),
    ("hvp_kernels.hip", []),
    ("api.hip", []),
    ("hvp_api.hip", []),
    ("cost_prep.hip", []),
    ("probe_kernels.hip", []),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libflashot.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    for name, extra in SOURCES:
        obj = os.path.join(BUILD_DIR, name + ".o")
        objs.append(obj)
        jobs.append([HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, name), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg:
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
