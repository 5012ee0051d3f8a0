"""Host-side logic of bench.py (no GPU): the HBM traffic figure is taken from
a committed counter summary only while the kernel sources it was measured on
are unchanged, and a multi-GPU request is refused before anything runs."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    csrc = tmp_path / "block_sparse_long_stride_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// kernel v1\n")
    (csrc / "h.h").write_text("// header\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _write_summary(root, source_hash, nbytes=123456789):
    rec = {"kernel": "k", "workload": "w", "sources": ["k.hip", "h.h"],
           "source_hash": source_hash, "bytes_per_launch": nbytes}
    (root / "profiles" / "traffic_k_w.json").write_text(json.dumps(rec))


def test_traffic_taken_when_sources_match(fake_root):
    _write_summary(fake_root, bench.kernel_source_hash(["k.hip", "h.h"]))
    assert bench.measured_traffic("k", "w") == 123456789


def test_traffic_dropped_after_a_kernel_change(fake_root):
    _write_summary(fake_root, bench.kernel_source_hash(["k.hip", "h.h"]))
    (fake_root / "block_sparse_long_stride_amd" / "csrc" / "k.hip").write_text("// kernel v2\n")
    assert bench.measured_traffic("k", "w") is None


def test_traffic_absent_without_summary(fake_root):
    assert bench.measured_traffic("k", "w") is None


def test_hash_depends_on_every_listed_source(fake_root):
    h = bench.kernel_source_hash(["k.hip", "h.h"])
    (fake_root / "block_sparse_long_stride_amd" / "csrc" / "h.h").write_text("// header v2\n")
    assert bench.kernel_source_hash(["k.hip", "h.h"]) != h


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_model_read_from_proc_cpuinfo():
    m = bench.cpu_model()
    if os.path.exists("/proc/cpuinfo"):
        assert isinstance(m, str) and m
