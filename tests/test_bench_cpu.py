"""bench.py's contract on the CPU: it runs on one GPU only (any other --gpus
exits with a message before touching a device), and the CPU baseline times the
oracle on a bounded sample and reports the fields the JSON line carries."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    for n in (2, 8):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=120)
        assert p.returncode == 2, p.stderr
        assert "one GPU" in p.stderr
        assert p.stdout == ""


def test_cpu_baseline_fields():
    import bench

    w = bench.make_workload("tiny")
    kv = 35 * 64 * 4 * 2  # the tiny workload's K/V bytes (35 fp32 rows of 64, K and V)
    r = bench.cpu_baseline(w, 0.2, kv)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] == 1
    assert r["value"] > 0 and r["rows_per_s"] > 0
    assert "whole decode rows" in r["sample"] and "binary64" in r["sample"]
