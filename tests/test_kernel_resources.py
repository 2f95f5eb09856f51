"""Compiler resource report of every kernel (no GPU needed): none may use
scratch memory, whose per-lane traffic would sit on the decode path as a
register spill or a stack frame of an out-of-line call."""
import shutil

import pytest

from memory_bound_decode_amd import _build


@pytest.fixture(scope="module")
def resources():
    if not (shutil.which("hipcc") or shutil.which("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    return _build.kernel_resources()


def test_every_source_reports_kernels(resources):
    names = " ".join(resources)
    for k in ("gemv_bn_kernel", "gemv_mq_kernel", "verify_gemm_kernel", "spec_gemv_kept_kernel", "enc_write_kernel"):
        assert k in names, k
    for r in resources.values():
        assert {"vgprs", "scratch", "occupancy"} <= set(r)


def test_no_kernel_uses_scratch(resources):
    bad = {n: r["scratch"] for n, r in resources.items() if r["scratch"] != 0}
    assert not bad, bad
