"""bench.py host logic on the CPU: the one-GPU guard and the committed HBM
traffic summary of the headline workload (it must describe the score kernel
as it stands, or the bench reports no traffic)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_summary_matches_kernel_sources():
    import bench
    t = bench.measured_traffic("fp8_128k_b32", 4000)
    assert t is not None, "profiles/ traffic summary is stale: re-run the FETCH/WRITE passes"
    # counters scaled by the copy calibration: within a few % of the algorithmic bytes
    assert 0.95 * 343158016 < t < 1.2 * 343158016


def test_traffic_summary_rejects_other_sources(tmp_path, monkeypatch):
    import bench
    monkeypatch.setattr(bench, "score_source_hash", lambda: "0000000000000000")
    assert bench.measured_traffic("fp8_128k_b32", 4000) is None
    assert bench.measured_traffic("no_such_workload", 4000) is None
