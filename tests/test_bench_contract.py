"""Host-side parts of bench.py (CPU only): one GPU only, and the counter-measured
traffic is reported only while the profile was taken on the current kernel
sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_traffic_is_read_only_for_the_profiled_sources(monkeypatch):
    d = bench.read_traffic("rec_kernel_decode_256x1tok")
    if d is not None:  # the profile matches the sources: its numbers are self-consistent
        assert d["bytes_per_launch"] == d["fetch_bytes"] + d["write_bytes"]
        assert 0.9 < d["bytes_per_launch"] / d["algorithmic_bytes"] < 1.2
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_traffic("rec_kernel_decode_256x1tok") is None
    assert bench.read_traffic("no_such_kernel") is None
