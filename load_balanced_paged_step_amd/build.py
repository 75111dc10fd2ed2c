"""Compile the decode library for gfx950 in-tree with hipcc.

Produces ``load_balanced_paged_step_amd/libhpc_decode.so`` (git-ignored; it
travels with the source tree).  Run ``python -m load_balanced_paged_step_amd.build``
or call :func:`build`.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libhpc_decode.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = [
    "csrc/plan.cpp",
    "csrc/api.cpp",
    "csrc/decode_kernels.hip",
    "csrc/probe_kernels.hip",
    "csrc/step_noalloc.hip",
    "csrc/prologue_api.cpp",
    "csrc/prologue_kernels.hip",
    "csrc/prefill_api.cpp",
    "csrc/prefill_kernels.hip",
]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"),
          "-I", os.path.join(HERE, "csrc")]
# Packed-fp32 VALU forms are kept out of the device code: the compiler may
# form them from plain float code, and they are avoided on these parts.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the decode library)")


def _rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(HERE, src)
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        if src.endswith(".hip"):
            cmd = [hipcc, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
        else:   # host-only C++ (still through hipcc for the HIP runtime headers)
            cmd = [hipcc, *COMMON, "-I", os.path.join(_rocm(), "include"), "-D__HIP_PLATFORM_AMD__",
                   "-x", "c++", "-c", path, "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
