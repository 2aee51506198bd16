"""Host logic of bench.py (no GPU): the one-GPU contract and the rule that
the PMC traffic figure is reported only for the kernel sources it was
measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_withheld_when_the_sources_differ(monkeypatch):
    monkeypatch.setattr(bench, "f1_source_hash", lambda: "0" * 64)
    assert bench.profiled_traffic() is None


def test_traffic_of_the_committed_profile():
    t = bench.profiled_traffic()
    if t is None:
        pytest.skip("the gate/up GEMV sources changed after its PMC traffic was taken")
    # measured HBM bytes per launch against 100 429 824 algorithmic bytes
    assert 100_429_824 <= t <= 1.01 * 100_429_824
