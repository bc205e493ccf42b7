"""Builds libcce.so (the gfx950 HIP kernels and the C ABI of include/cce.h) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcce.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libcce)")


def sources() -> list[str]:
    """Every HIP translation unit of the library (csrc/*.hip)."""
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def compile_command(out: str) -> list[str]:
    # -packed-fp32-ops: the gfx950 code generator emits no packed fp32 VALU forms (scalar fp32
    # math only).  The device pass honours it; hipcc's host pass, which compiles the same files
    # for x86, prints that it does not know the feature, which is harmless.
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"), *sources(), "-o", out]


def build(verbose: bool = False) -> str:
    """Compile libcce.so next to this file (always recompiles); returns its path."""
    tmp = LIB + ".tmp"
    cmd = compile_command(tmp)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libcce build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
