"""Host-side behaviour of bench.py that needs no GPU: the one-GPU contract and the rule
that stored HBM-traffic counts are reported only for the kernel source they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fake_tree(tmp_path, source_text):
    for f in bench.KERNEL_SOURCES:
        p = tmp_path / f
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text(source_text)
    (tmp_path / "profiles").mkdir(exist_ok=True)


def test_traffic_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _fake_tree(tmp_path, "kernel v1")
    h1 = bench.kernel_source_hash()
    entry = {"bytes_per_launch": 123456.0}
    (tmp_path / "profiles" / "traffic.json").write_text(
        json.dumps({"source_sha256": h1, "shapes": {"shape_a": entry}}))
    assert bench.load_traffic("shape_a") == 123456.0
    assert bench.load_traffic("shape_b") is None
    _fake_tree(tmp_path, "kernel v2")                  # the kernel changed since
    assert bench.kernel_source_hash() != h1
    assert bench.load_traffic("shape_a") is None


def test_traffic_absent_or_unreadable(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _fake_tree(tmp_path, "kernel")
    assert bench.load_traffic("shape_a") is None
    (tmp_path / "profiles" / "traffic.json").write_text("{not json")
    assert bench.load_traffic("shape_a") is None
