"""bench.py on the CPU: the multi-GPU request is refused before any device is
touched, and the stored HBM-traffic record is tied to the kernel source and
launch configuration it was measured on."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_applies_only_to_its_source_and_launch(monkeypatch):
    """The stored counter bytes are reported for the kernel source and the
    launch configuration they were measured on, and for nothing else."""
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "decode_traffic.json")) as f:
        rec = json.load(f)
    key = rec["config"]
    monkeypatch.setattr(bench, "source_hash", lambda: rec["kernel_source_sha256_16"])
    t = bench.stored_traffic(key)
    assert t is not None and t > 75497472  # at least the default workload's cache stream
    other = dict(key, workload="long_b4_l32k", splits=64)
    assert bench.stored_traffic(other) is None
    assert bench.stored_traffic(dict(key, decode_kernel="h128")) is None
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.stored_traffic(key) is None
