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


def test_profile_digest_ignores_comments_only():
    """A profile's traffic is read only while the decode code it measured is
    unchanged: the digest ignores comments and whitespace and sees any code
    edit.  Every committed decode profile carries one."""
    import glob
    import re
    import shutil
    import tempfile

    import bench

    tmp = tempfile.mkdtemp()
    try:
        src = os.path.join(ROOT, "block_table_attention_amd", "csrc")
        dst = os.path.join(tmp, "block_table_attention_amd", "csrc")
        os.makedirs(dst)
        for f in ("paged_decode.hip", "pba_internal.h"):
            shutil.copy(os.path.join(src, f), dst)
        base = bench.decode_source_digest(tmp)
        path = os.path.join(dst, "paged_decode.hip")
        text = open(path).read()
        open(path, "w").write("// a note\n/* and a block\n comment */\n" + text.replace("\n", "\n  "))
        assert bench.decode_source_digest(tmp) == base
        open(path, "w").write(text + "\nconstexpr int kAnotherConstant = 1;\n")
        assert bench.decode_source_digest(tmp) != base
    finally:
        shutil.rmtree(tmp)
    files = glob.glob(os.path.join(ROOT, "profiles", "decode_bf16_*.md"))
    assert files
    for f in files:
        assert re.search(r"decode_code_sha256: [0-9a-f]{64}", open(f).read()), f
