"""Host-side parts of bench.py (no GPU): the one-GPU guard, the rule that stored
HBM counters apply only to the kernel source they were taken on, the CPU
baseline record, and the arithmetic of the committed counter summary."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


class _Wl:
    name = "toy_workload"

    def __init__(self):
        self.calls = 0

    def oracle_call(self):
        self.calls += 1
        return self.calls

    def bytes_per_step(self):
        return 1000


def _fake_tree(tmp_path, gemv_text):
    csrc = tmp_path / "memory_bound_decode_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "gemv.hip").write_text(gemv_text)
    (csrc / "mbd_internal.h").write_text("// header\n")
    (tmp_path / "profiles").mkdir()


def test_traffic_applies_only_to_its_source(tmp_path, monkeypatch):
    _fake_tree(tmp_path, "kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    wl = _Wl()
    assert bench.traffic_from_profiles(wl) is None                     # no summary
    rec = {"source_sha256": bench.source_hash(), "hbm_bytes_per_step": 12345}
    (tmp_path / "profiles" / "toy_workload_traffic.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles(wl) == 12345
    (tmp_path / "memory_bound_decode_amd" / "csrc" / "gemv.hip").write_text("kernel v2\n")
    assert bench.traffic_from_profiles(wl) is None                     # kernel changed since


def test_cpu_baseline_record():
    wl = _Wl()
    rec, ref = bench.cpu_baseline(wl, budget_s=0.01)
    assert ref == 1 and wl.calls >= 1
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s"
    assert rec["cores"] >= 1 and rec["value"] > 0
    assert "oracle" in rec["sample"] and wl.name in rec["sample"]


def test_committed_traffic_summary_is_consistent():
    path = os.path.join(ROOT, "profiles", "int4_g128_gemv_8192x8192_b1_traffic.json")
    if not os.path.exists(path):
        pytest.skip("no committed counter summary")
    d = json.load(open(path))
    # scales: the copy kernel's bytes over what its counters read
    assert d["fetch_scale"] == pytest.approx(d["copy_kernel_bytes"] / 1024 / d["copy_fetch_kib"], rel=1e-3)
    assert d["write_scale"] == pytest.approx(d["copy_kernel_bytes"] / 1024 / d["copy_write_kib"], rel=1e-3)
    hbm = (d["fetch_kib_per_dispatch"] * d["fetch_scale"] + d["write_kib_per_dispatch"] * d["write_scale"]) * 1024
    assert d["hbm_bytes_per_step"] == pytest.approx(hbm, rel=1e-3)
    assert d["ratio"] == pytest.approx(d["hbm_bytes_per_step"] / d["algorithmic_bytes_per_step"], rel=1e-3)
    # INT4 8192 x 8192: codes + fp16 scales + bf16 x + fp32 y
    assert d["algorithmic_bytes_per_step"] == 8192 * 8192 // 2 + 8192 * 64 * 2 + 8192 * 2 + 8192 * 4
