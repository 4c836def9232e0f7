"""bench.py's command-line contract on the CPU: one GPU only (a request for
more exits with status 2 and a message, before any device is touched), and
the stored GEMM traffic figure is tied to the GEMM sources and the rank it
was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout.strip() == ""


def test_traffic_figure_follows_the_gemm_sources(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    assert bench.gemm_traffic() == bench.GEMM_TRAFFIC_BYTES
    monkeypatch.setattr(bench, "GEMM_TRAFFIC_SHA1", "0" * 40)
    assert bench.gemm_traffic() is None


def test_traffic_figure_is_for_rank_64(monkeypatch):
    """The stored counter figure was taken at r = 64: other ranks report none."""
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(bench, "R", 8)
    assert bench.gemm_traffic() is None
    monkeypatch.setattr(bench, "R", 64)
    assert bench.gemm_traffic() == bench.GEMM_TRAFFIC_BYTES
