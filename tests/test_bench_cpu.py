"""bench.py's host-side contract (no GPU needed)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import bench
from dense_gemm_09_amd import roofline

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_peaks_come_from_the_roofline_module():
    assert bench.PEAK["bf16"] == roofline.MI355X_PEAK_TFLOPS["bf16"]
    assert bench.PEAK["fp8"] == roofline.MI355X_PEAK_TFLOPS["fp8"]
    assert bench.HBM_GBPS == roofline.MI355X_HBM_GBPS


def test_source_hash_covers_every_library_source(tmp_path, monkeypatch):
    """Changing any file under csrc/ or include/ changes the hash that decides
    whether a committed counter profile still describes the kernels."""
    root = tmp_path / "tree"
    shutil.copytree(os.path.join(ROOT, "dense_gemm_09_amd", "csrc"),
                    root / "dense_gemm_09_amd" / "csrc")
    shutil.copytree(os.path.join(ROOT, "include"), root / "include")
    monkeypatch.setattr(bench, "ROOT", str(root))
    base = bench.kernel_source_sha()
    files = sorted(p for p in root.rglob("*") if p.suffix in (".hip", ".hpp", ".cpp", ".h"))
    assert len(files) >= 6
    for path in files:
        old = path.read_bytes()
        path.write_bytes(old + b"\n")
        assert bench.kernel_source_sha() != base, path.name
        path.write_bytes(old)
    assert bench.kernel_source_sha() == base


def test_traffic_is_reported_only_for_the_profiled_source(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.measured_traffic() is None
