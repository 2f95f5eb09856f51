"""The C++ packer (every format, the section / statistics / validation calls and
their error paths) and the host side of every C-ABI entry point (argument checks,
error reporting, size arithmetic) under AddressSanitizer and UndefinedBehavior-
Sanitizer: host builds with tests/sanitize/packer_driver.cpp and
tests/sanitize/abi_driver.cpp, run here on the CPU; any sanitizer report fails the
test."""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "memory_bound_decode_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_packer_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "packer_driver")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               os.path.join(CSRC, "packer.cpp"), os.path.join(ROOT, "tests", "sanitize", "packer_driver.cpp"),
               "-o", exe, "-lpthread"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        env.pop("LD_PRELOAD", None)
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
        assert "all checks passed" in r.stdout


HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
def test_abi_host_code_under_asan_ubsan():
    """The library's HIP sources with only their host passes instrumented (the device
    code is built but never run: every call in the driver fails validation before any
    launch), linked with the packer and the driver, one clang sanitizer runtime."""
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    host_san = []
    for f in san:
        host_san += ["-Xarch_host", f]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory() as td:
        cmds = []
        objs = []
        for src in ("gemv.hip", "cassandra.hip", "encoder.hip", "probe.hip"):
            o = os.path.join(td, src + ".o")
            objs.append(o)
            cmds.append([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, *inc,
                         "-c", os.path.join(CSRC, src), "-o", o])
        for src in (os.path.join(CSRC, "packer.cpp"), os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")):
            o = os.path.join(td, os.path.basename(src) + ".o")
            objs.append(o)
            cmds.append([CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *san, *inc, "-c", src, "-o", o])
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
        for c, r in zip(cmds, results):
            assert r.returncode == 0, (" ".join(c[-3:]), r.stderr[-3000:])
        exe = os.path.join(td, "abi_driver")
        r = subprocess.run([HIPCC, *san, "-o", exe, *objs, "-lpthread"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        env.pop("LD_PRELOAD", None)
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
        assert r.stdout.strip() == "ok"
