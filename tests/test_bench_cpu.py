"""bench.py's host-side contract (no GPU): one GPU only, with a message for
any other count, and the recorded GEMM traffic is used only while the GEMM
sources are the ones the counters were taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_follows_the_gemm_sources(monkeypatch):
    import bench
    assert bench.gemm_traffic_bytes() is not None          # the committed record matches the sources
    rec = dict(bench.GEMM_TRAFFIC, source_sha256="0" * 64)
    monkeypatch.setattr(bench, "GEMM_TRAFFIC", rec)
    assert bench.gemm_traffic_bytes() is None
