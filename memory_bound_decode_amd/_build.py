"""Build libmbd.so in-tree: the C++ packer with g++, the HIP kernels with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libmbd.so")

HIP_SOURCES = ["gemv.hip", "cassandra.hip", "encoder.hip"]
CXX_SOURCES = ["packer.cpp"]
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # never let the compiler form packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link libmbd.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    objs = []
    for s in CXX_SOURCES:
        o = os.path.join(OBJ, s + ".o")
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    hipcc = _hipcc()
    for s in HIP_SOURCES:
        o = os.path.join(OBJ, s + ".o")
        _run([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
