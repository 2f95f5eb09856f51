"""Build libmbd.so in-tree: the C++ packer with g++, the HIP kernels with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libmbd.so")

HIP_SOURCES = ["gemv.hip", "cassandra.hip", "encoder.hip", "probe.hip"]
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


def _run_all(cmds):
    """Run the compile commands side by side; raise on the first that failed."""
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)) for c in cmds]
    outs = [(c, p.communicate(), p.returncode) for c, p in procs]
    for c, (out, err), rc in outs:
        if rc != 0:
            raise RuntimeError("build step failed: %s\n%s%s" % (" ".join(c), out, err))


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link libmbd.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    hipcc = _hipcc()
    cmds, objs = [], []
    for s in CXX_SOURCES:
        objs.append(os.path.join(OBJ, s + ".o"))
        cmds.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", objs[-1]])
    for s in HIP_SOURCES:
        objs.append(os.path.join(OBJ, s + ".o"))
        cmds.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", objs[-1]])
    _run_all(cmds)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)


def kernel_resources() -> dict:
    """Per-kernel register, scratch and occupancy figures the compiler reports for
    every HIP source (a device-only compile with the build's flags):
    {mangled name: {"vgprs": n, "scratch": bytes per lane, "occupancy": waves per SIMD}}."""
    import re
    import tempfile
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory() as td:
        cmds = [[hipcc, *HIPCC_FLAGS, "--cuda-device-only", "-c", os.path.join(CSRC, s),
                 "-o", os.path.join(td, s + ".o"), "-Rpass-analysis=kernel-resource-usage"] for s in HIP_SOURCES]
        procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True) for c in cmds]
        texts = []
        for c, p in zip(cmds, procs):
            out, err = p.communicate()
            if p.returncode != 0:
                raise RuntimeError("compile failed: %s\n%s" % (" ".join(c), err))
            texts.append(err)
    res, cur = {}, None
    for line in "\n".join(texts).splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = res.setdefault(m.group(1), {})
            continue
        for key, pat in (("vgprs", r"\bVGPRs: (\d+)"), ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                         ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(pat, line)
            if m and cur is not None:
                cur[key] = int(m.group(1))
    return res
