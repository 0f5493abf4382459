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


def test_counter_record_applies_only_to_its_source_and_launch(monkeypatch, tmp_path):
    """A stored counter record is reported for the kernel source and the launch
    configuration it was measured on, and for nothing else; records of several
    configurations live side by side."""
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "decode_traffic.json")) as f:
        recs = json.load(f)["records"]
    assert recs and all("config" in r and "hbm_bytes_per_launch" in r for r in recs)
    a = bench.traffic_key("paged_b64_ragged", 8, "bf16", "auto")
    b = bench.traffic_key("long_b4_l32k", 64, "bf16", "auto")
    store = tmp_path / "t.json"
    json.dump({"records": [dict(config=a, kernel_source_sha256_16="1" * 16, hbm_bytes_per_launch=7.0),
                           dict(config=b, kernel_source_sha256_16="1" * 16, hbm_bytes_per_launch=9.0)]},
              open(store, "w"))
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(store))
    monkeypatch.setattr(bench, "source_hash", lambda: "1" * 16)
    assert bench.stored_counters(a)["hbm_bytes_per_launch"] == 7.0
    assert bench.stored_counters(b)["hbm_bytes_per_launch"] == 9.0
    assert bench.stored_counters(dict(a, decode_kernel="h64")) is None
    assert bench.stored_counters(dict(a, splits=16)) is None
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.stored_counters(a) is None


def test_launch_stats():
    sys.path.insert(0, ROOT)
    import bench
    st = bench.launch_stats([float(x) for x in range(1, 102)])
    assert st["median"] == 51.0 and st["p10"] == 11.0 and st["p90"] == 91.0
    assert st["mean"] == 51.0 and st["n"] == 101


def test_one_thread_oracle_baseline():
    """the one-thread oracle timing runs in a child process with one OpenMP
    thread and reports it"""
    sys.path.insert(0, ROOT)
    import bench
    r = bench.cpu_baseline_one_core("tiny_f32", 0.1)
    assert r["cores"] == 1 and r["kind"] == "oracle" and r["value"] > 0
    assert "one host thread" in r["sample"]
