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
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["cores"] == len(os.sched_getaffinity(0))
    assert r["cpu_model"] and r["cpu_model"] != "unknown"
    assert r["value"] > 0 and r["rows_per_s"] > 0
    assert r["value_1_thread"] > 0 and r["rows_per_s_1_thread"] > 0
    assert "whole decode rows" in r["sample"] and "binary64" in r["sample"]


def _digest_tree(tmp):
    import shutil

    import bench

    for rel in bench.DIGEST_SOURCES:
        src = os.path.join(ROOT, rel)
        if os.path.exists(src):
            os.makedirs(os.path.dirname(os.path.join(tmp, rel)), exist_ok=True)
            shutil.copy(src, os.path.join(tmp, rel))


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
        _digest_tree(tmp)
        base = bench.decode_source_digest(tmp)
        path = os.path.join(tmp, "block_table_attention_amd", "csrc", "paged_decode.hip")
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


def test_planner_edit_voids_profiled_traffic():
    """The traffic figure of a profile is tied to the planners too: an edit to
    the library's partition planner or to the caller-side partition helper
    makes profiled_traffic return None (roofline.traffic null)."""
    import shutil
    import tempfile

    import bench

    tmp = tempfile.mkdtemp()
    try:
        _digest_tree(tmp)
        os.makedirs(os.path.join(tmp, "profiles"))
        prof = os.path.join(tmp, "profiles", "decode_bf16_long16k.md")
        open(prof, "w").write(f"    traffic_bytes_per_launch: 1234\n"
                              f"    decode_code_sha256: {bench.decode_source_digest(tmp)}\n")
        assert bench.profiled_traffic("long16k", tmp) == 1234
        for rel, edit in (("block_table_attention_amd/csrc/pba_api.hip",
                           "\nstatic int planner_edit = 2;\n"),
                          ("block_table_attention_amd/blocks.py", "\nPLANNER_EDIT = 2\n")):
            path = os.path.join(tmp, rel)
            text = open(path).read()
            open(path, "a").write("# a comment only\n" if rel.endswith(".py") else "// a comment only\n")
            assert bench.profiled_traffic("long16k", tmp) == 1234, rel
            open(path, "w").write(text + edit)
            assert bench.profiled_traffic("long16k", tmp) is None, rel
            open(path, "w").write(text)
            assert bench.profiled_traffic("long16k", tmp) == 1234, rel
    finally:
        shutil.rmtree(tmp)


def test_fused_step_eligibility():
    """The bench fuses the step's appends into the decode call only when every
    new token is its row's last position in a block no other row reads, and,
    under a shared-prefix plan, inside its row's private range."""
    import numpy as np

    import bench
    from block_table_attention_amd.blocks import shared_plan, sharing_order

    w = bench.make_workload("long16k")
    plan = bench.plan_script(w)
    assert bench.step_rows_if_fusable(plan, 64) == list(range(8))

    w = bench.make_workload("shared_prefix")
    plan = bench.plan_script(w)
    rows = bench.step_rows_if_fusable(plan, 16)
    assert rows is not None and len(rows) == 64 and len(plan.step_src) > 0
    order = sharing_order(plan.tables)
    lens = plan.seq_lens[order]
    hp = shared_plan(plan.tables[order], lens, 16, 4, 1024, tiles_per_item=2)
    srows = bench.shared_step_rows(rows, order, hp, lens)
    assert srows is not None and sorted(order[srows].tolist()) == sorted(rows)
    # A plan whose range starts past a new token: the token would sit in a chunk.
    hp.row_private = hp.row_private.copy()
    hp.row_private[srows[0], 0] = lens[srows[0]]
    assert bench.shared_step_rows(rows, order, hp, lens) is None

    def plan_of(tables, lens, slots):
        t = np.array(tables, np.int32)
        return bench.Plan([], np.zeros(0, np.int32), np.zeros(0, np.int32),
                          np.array(slots, np.int64), (0, len(slots)), t,
                          np.array(lens, np.int32), len(slots))

    # Two rows ending in one block (a fork that has not written yet): no.
    assert bench.step_rows_if_fusable(plan_of([[4, 5], [4, 5]], [20, 20], [5 * 16 + 3]), 16) is None
    # Row 1 reads row 0's last block: no.
    assert bench.step_rows_if_fusable(plan_of([[4, 5], [5, 6]], [20, 20], [5 * 16 + 3]), 16) is None
    # A slot that is not a last position: no.  Each row alone: yes.
    assert bench.step_rows_if_fusable(plan_of([[4, 5], [7, 6]], [20, 20], [5 * 16 + 2]), 16) is None
    assert bench.step_rows_if_fusable(plan_of([[4, 5], [7, 6]], [20, 20], [6 * 16 + 3, 5 * 16 + 3]),
                                      16) == [1, 0]
