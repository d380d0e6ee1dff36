"""CPU checks of bench.py's contract that need no GPU: more than one GPU is refused
with a message (this library measures one GPU), and the traffic figure is read
from the committed counter summary only while the kernel sources match it."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_tied_to_the_kernel_sources(tmp_path, monkeypatch):
    # the committed summary matches the current sources
    t = bench.measured_traffic()
    assert t is not None and t > 0
    # a summary recorded for other sources is ignored
    fake = tmp_path / "traffic.md"
    fake.write_text("kernel-source-hash: 0000000000000000\ntraffic-per-launch-bytes: 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(fake))
    assert bench.measured_traffic() is None
    # a missing summary gives no figure
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None
