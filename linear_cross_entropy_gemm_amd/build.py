"""Build ``libflce.so`` in-tree with hipcc for gfx950.

Usage: ``python linear_cross_entropy_gemm_amd/build.py`` (run by path: importing the
package loads the library, which may not exist or may be stale).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libflce.so")

SOURCES = ["flce_kernels.hip", "flce_logits.hip", "flce_scale.hip", "flce_noalloc.hip", "flce_plan.cpp",
           "flce_api.cpp", "flce_profile.cpp"]
HEADERS = ["device_common.hpp", "gemm_tile.hpp", "flce_internal.hpp", "kernel_args.hpp"]

ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code (the compiler would
# otherwise form v_pk_* from plain float code).
# -packed-fp32-ops: no packed fp32 VALU; -ffp-contract=off: the kernels spell
# out every fused multiply-add, so the same expression rounds the same way in
# every instantiation (the forward-only entry reproduces the full call bitwise)
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the FLCE library)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source into ``libflce.so`` (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", *DEVICE_FLAGS,
           "-I", os.path.join(ROOT, "include"),
           *(extra_flags or []),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
