"""Host logic of bench.py (no GPU): the one-GPU contract and the traffic file check."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_for_its_workload_and_kernel_source(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()
    f = tmp_path / "traffic.txt"
    f.write_text(f"# comment: ignored\nkernel_source_sha: {sha}\nworkload: w1\nhbm_bytes_per_launch: 123.5\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic("w1") == 123.5
    assert bench.read_traffic("w2") is None                 # another workload
    f.write_text("kernel_source_sha: 0000000000000000\nworkload: w1\nhbm_bytes_per_launch: 123.5\n")
    assert bench.read_traffic("w1") is None                 # taken from an older kernel source
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic("w1") is None


def test_committed_traffic_matches_the_current_step_kernel():
    # the committed counter summary was taken from this kernel source on the default workload
    assert bench.read_traffic(bench.DEFAULT_WORKLOAD) is not None
