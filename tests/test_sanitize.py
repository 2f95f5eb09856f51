"""The C++ packer (every format, the section / statistics / validation calls and
their error paths) under AddressSanitizer and UndefinedBehaviorSanitizer: a host
build of packer.cpp with tests/sanitize/packer_driver.cpp, compiled with g++ and
run here on the CPU; any sanitizer report fails the test."""
import os
import shutil
import subprocess
import tempfile

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
