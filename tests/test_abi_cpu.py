"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad host-visible arguments before any launch."""
import ctypes
import os
import re

import pytest

from conftest import ROOT


def _header_functions():
    with open(os.path.join(ROOT, "include", "pba.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(pba_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported():
    import block_table_attention_amd as pba

    lib = ctypes.CDLL(pba.lib_path())
    declared = _header_functions()
    assert declared == sorted(pba.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert pba.version() == 400


def _desc(**kw):
    import block_table_attention_amd as pba

    d = dict(k=0x10000, v=0x20000, dtype=1, num_blocks=8, block_size=16, num_kv_heads=2,
             head_dim=128, split_log2=0, k_stride_block=2 * 16 * 128, k_stride_head=16 * 128,
             v_stride_block=2 * 16 * 128, v_stride_head=16 * 128)
    d.update(kw)
    return pba.PoolDesc(**d)


def _lib():
    import block_table_attention_amd as pba
    return pba._lib


NULL = None


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), -2),
    (dict(block_size=48), -4),
    (dict(block_size=8), -4),
    (dict(block_size=512), -4),
    (dict(head_dim=96), -4),
    (dict(num_blocks=0), -3),
    (dict(num_kv_heads=0), -3),
    (dict(split_log2=-1), -3),
    (dict(split_log2=5), -4),
    (dict(split_log2=1, num_blocks=7), -3),       # kernel blocks not a multiple of q
    (dict(k=0), -1),
    (dict(k=0x10008), -4),
    (dict(k_stride_head=1024), -3),
    (dict(k_stride_head=16 * 128 + 4), -4),
    (dict(v_stride_block=-16), -3),
])
def test_pool_descriptor_rejections(kw, status):
    lib = _lib()
    d = _desc(**kw)
    assert lib.pba_kv_append(ctypes.byref(d), 0x30000, 4, 0x40000, 0x50000, NULL) == status
    assert lib.pba_block_copy(ctypes.byref(d), 0x30000, 0x30010, 4, NULL) == status
    assert lib.pba_paged_decode(ctypes.byref(d), 0x30000, 8, 0x40000, 4, 0x50000, 2,
                                ctypes.c_float(0.1), 0x60000, NULL, 0, 0x70000, 1 << 30, NULL) == status


def test_null_pool_and_pointers():
    lib = _lib()
    assert lib.pba_kv_append(NULL, 0x30000, 4, 0x40000, 0x50000, NULL) == -1
    d = _desc()
    assert lib.pba_kv_append(ctypes.byref(d), NULL, 4, 0x40000, 0x50000, NULL) == -1
    assert lib.pba_block_copy(ctypes.byref(d), NULL, 0x30000, 1, NULL) == -1
    assert lib.pba_paged_decode(ctypes.byref(d), NULL, 8, 0x40000, 4, 0x50000, 2,
                                ctypes.c_float(0.1), 0x60000, NULL, 0, NULL, 0, NULL) == -1


def test_empty_calls_are_noops():
    lib = _lib()
    d = _desc()
    assert lib.pba_kv_append(ctypes.byref(d), NULL, 0, NULL, NULL, NULL) == 0
    assert lib.pba_block_copy(ctypes.byref(d), NULL, NULL, 0, NULL) == 0
    assert lib.pba_paged_decode(ctypes.byref(d), NULL, 8, NULL, 4, NULL, 0,
                                ctypes.c_float(0.1), NULL, NULL, 0, NULL, 0, NULL) == 0
    assert lib.pba_kv_append(ctypes.byref(d), NULL, -1, NULL, NULL, NULL) == -3


def test_decode_shape_rejections():
    lib = _lib()
    d = _desc()
    call = lambda hq, mb, pt, ws, wsb: lib.pba_paged_decode(
        ctypes.byref(d), 0x30000, hq, 0x40000, mb, 0x50000, 2, ctypes.c_float(0.1), 0x60000,
        NULL, pt, ws, wsb, NULL)
    assert call(7, 4, 0, NULL, 0) == -3          # H_q not a multiple of H_kv
    assert call(34, 4, 0, NULL, 0) == -4         # G = 17 > 16
    assert call(8, 0, 0, NULL, 0) == -3          # no table width
    assert call(8, 64, 100, NULL, 0) == -4       # partition not a multiple of 256
    assert call(8, 64, -256, NULL, 0) == -3
    # 64 blocks * 16 = 1024 tokens in 256-token partitions -> 4 partitions need a workspace.
    assert call(8, 64, 256, NULL, 0) == -5
    need = lib.pba_paged_decode_workspace_bytes(ctypes.byref(d), 8, 2, 64, 256)
    assert call(8, 64, 256, 0x80000, need - 1) == -5
    assert call(8, 64, 256, 0x80008, need) == -5  # misaligned workspace
    # q is read in 16-byte pieces.
    assert lib.pba_paged_decode(ctypes.byref(d), 0x30008, 8, 0x40000, 4, 0x50000, 2,
                                ctypes.c_float(0.1), 0x60000, NULL, 0, NULL, 0, NULL) == -4


def test_decode_stride_limit():
    """The decode kernel takes the K strides as int32: larger ones are rejected
    by all three decode entry points, while append and copy accept them."""
    lib = _lib()
    big = _desc(k_stride_block=1 << 31)
    pt, npart = ctypes.c_int32(), ctypes.c_int32()
    assert lib.pba_paged_decode(ctypes.byref(big), 0x30000, 8, 0x40000, 4, 0x50000, 2,
                                ctypes.c_float(0.1), 0x60000, NULL, 0, NULL, 0, NULL) == -4
    assert lib.pba_paged_decode_plan(ctypes.byref(big), 8, 2, 4, 0, ctypes.byref(pt),
                                     ctypes.byref(npart)) == -4
    assert lib.pba_paged_decode_workspace_bytes(ctypes.byref(big), 8, 2, 64, 256) == 0
    assert lib.pba_kv_append(ctypes.byref(big), NULL, 0, NULL, NULL, NULL) == 0


def test_workspace_and_plan():
    import block_table_attention_amd as pba

    lib = _lib()
    d = _desc()
    pt, npart = ctypes.c_int32(), ctypes.c_int32()
    assert lib.pba_paged_decode_plan(ctypes.byref(d), 8, 2, 64, 256, ctypes.byref(pt), ctypes.byref(npart)) == 0
    assert (pt.value, npart.value) == (256, 4)
    rows = 2 * 8
    up = lambda x: (x + 255) // 256 * 256
    counters = 2 * 2 * 4                     # B * H_kv int32
    ml = rows * 4 * 2 * 4                    # rows * n_parts * (m, l)
    expect = up(counters) + up(ml) + rows * 4 * 128 * 4
    assert lib.pba_paged_decode_workspace_bytes(ctypes.byref(d), 8, 2, 64, 256) == expect
    # A single partition needs no workspace.
    assert lib.pba_paged_decode_workspace_bytes(ctypes.byref(d), 8, 2, 64, 1024) == 0
    # T = 2049 in 512-token partitions -> 5 (the pages' fixture), P = 16 -> 129 blocks.
    assert lib.pba_paged_decode_plan(ctypes.byref(d), 8, 1, 129, 512, ctypes.byref(pt), ctypes.byref(npart)) == 0
    assert npart.value == 5
    # Automatic plans: partitions are multiples of 256 and cover the table.
    # PBA_PARTITIONS_BALANCED falls back to them where the balanced decode
    # does not apply (fp32 pools, batches over 2048 rows).
    f32 = _desc(dtype=0)
    for desc, B, mb, req in [(d, 1, 1, 0), (d, 8, 256, 0), (d, 32, 129, 0), (d, 1, 4096, 0),
                             (d, 128, 512, 0), (f32, 8, 256, -1), (d, 4096, 8, -1)]:
        assert lib.pba_paged_decode_plan(ctypes.byref(desc), 8, B, mb, req, ctypes.byref(pt),
                                         ctypes.byref(npart)) == 0
        assert pt.value % 128 == 0 and pt.value * npart.value >= mb * 16
        assert pt.value * (npart.value - 1) < mb * 16
    # The balanced decode: one 4-wave work-group per CU (256 CUs when no device
    # is visible); workspace = counters + two piece states per work-group (the
    # waves' pieces stay in LDS).
    for B, mb in [(1, 1), (8, 256), (2048, 4)]:
        assert lib.pba_paged_decode_plan(ctypes.byref(d), 8, B, mb, -1, ctypes.byref(pt),
                                         ctypes.byref(npart)) == 0
        waves = npart.value
        assert pt.value == 0 and waves % 4 == 0 and waves >= 4
        G, slots = 4, 2 * (waves // 4)
        expect = up(B * 2 * 4) + up(slots * G * 2 * 4) + slots * G * 128 * 4
        assert lib.pba_paged_decode_workspace_bytes(ctypes.byref(d), 8, B, mb, -1) == expect
    # Its LDS holds 8 wave pieces of G x (head_dim + 2) floats and the row
    # prefix sums, at most 64 KiB: G = 16 at head_dim 128 takes the grid plan,
    # head_dim 64 stays balanced up to 2048 rows.
    assert lib.pba_paged_decode_plan(ctypes.byref(d), 32, 8, 64, -1, ctypes.byref(pt),
                                     ctypes.byref(npart)) == 0
    assert pt.value > 0
    d64 = _desc(head_dim=64, k_stride_block=2 * 16 * 64, k_stride_head=16 * 64,
                v_stride_block=2 * 16 * 64, v_stride_head=16 * 64)
    assert lib.pba_paged_decode_plan(ctypes.byref(d64), 32, 2048, 4, -1, ctypes.byref(pt),
                                     ctypes.byref(npart)) == 0
    assert pt.value == 0
    assert lib.pba_paged_decode_plan(ctypes.byref(d), 8, 2, 64, -2, ctypes.byref(pt),
                                     ctypes.byref(npart)) == -3
    assert lib.pba_status_string(-5).decode().startswith("workspace")
    assert pba.STATUS[-6] == "PBA_ERR_OUT_OF_RANGE"


def test_validate_flag_roundtrip():
    import block_table_attention_amd as pba

    assert pba.set_validate(True) is False
    assert pba.set_validate(False) is True


@pytest.mark.parametrize("name", ["long16k", "batch32", "shared_prefix", "lognormal_p64", "tiny"])
def test_bench_plan_matches_oracle_allocator(name):
    """bench.py runs each workload script through the package's BlockManager;
    the tables, lengths, setup calls and step calls must be exactly the
    oracle allocator's trace for the same script (same slots, same copy pairs,
    same K/V rows), and the byte counts must follow from the tables."""
    import numpy as np

    import bench
    from harness import execute

    w = bench.make_workload(name)
    plan = bench.plan_script(w)
    ex = execute(w)
    assert np.array_equal(plan.tables, ex.tables)
    assert np.array_equal(plan.seq_lens, ex.seq_lens)
    assert plan.n_writes == ex.n_writes
    # Flatten both traces to (kind, payload) in program order.
    mine = []
    for op in plan.setup:
        if op[0] == "copy":
            mine += [("copy", int(s), int(d)) for s, d in zip(op[1], op[2])]
        else:
            mine += [("write", int(s), r) for s, r in zip(op[1], range(op[2], op[3]))]
    lo, hi = plan.step_rows
    assert hi - lo == len(plan.step_slots)
    step = [("copy", int(s), int(d)) for s, d in zip(plan.step_src, plan.step_dst)]
    step += [("write", int(s), r) for s, r in zip(plan.step_slots, range(lo, hi))]
    theirs = []
    for op in ex.ops:
        if op[0] == "copy":
            theirs += [("copy", int(s), int(d)) for s, d in zip(op[1], op[2])]
        else:
            theirs += [("write", int(s), r) for s, r in zip(op[1], range(op[2], op[3]))]
    # The step batches its copies ahead of its writes; the oracle interleaves
    # them per request.  Same multiset, and every copy precedes the writes
    # into its destination block in both.
    n_setup = len(mine)
    assert theirs[:n_setup] == mine
    assert sorted(theirs[n_setup:]) == sorted(step)
    P = w.shape.block_size
    # Batching is exact only if no step write lands in a block a step copy
    # reads (a copy then sees the same bytes in either order).
    src_blocks = {c[1] for c in step if c[0] == "copy"}
    assert all(op[1] // P not in src_blocks for op in step if op[0] == "write")
    kv_unique, kv_logical, alg = bench.decode_bytes(plan, w.shape)
    es = 2 if w.shape.dtype == "bf16" else 4
    row = w.shape.num_kv_heads * w.shape.head_dim * 2 * es
    assert kv_logical == int(ex.seq_lens.sum()) * row
    assert kv_unique <= kv_logical
    if name != "shared_prefix":
        assert kv_unique == kv_logical
    else:
        # The 2000-token prefix is read once by the 128 rows that map it.
        assert kv_logical - kv_unique >= 2000 * 127 * row


@pytest.mark.parametrize("name", ["lognormal_p16", "lognormal_p64", "lognormal_p256", "batch32"])
def test_bench_ledger_matches_oracle(name):
    """The bench's block-size accounting equals the oracle's ledgers (request
    view tail slots, dense and used table cells) for the same decode batch."""
    import bench
    from oracle import ledgers

    w = bench.make_workload(name)
    plan = bench.plan_script(w)
    P = w.shape.block_size
    got = bench.table_ledger(plan, P)
    lens = [int(T) for T in plan.seq_lens]
    view = ledgers.request_view_ledger(lens, P)
    cells = ledgers.table_cells(lens, P)
    assert got["tail_slots"] == view["tail_slots"]
    assert got["blocks_mapped"] == view["refs"] == cells["used"]
    assert got["table_cells_dense"] == cells["table"]


def test_shared_decode_host_rejections():
    """Host-side checks of pba_paged_decode_shared: fp32 pools, a missing or
    malformed plan, and partition lengths that are not multiples of 256 are
    rejected before any launch; the workspace size follows max_slots."""
    import block_table_attention_amd as pba

    lib = _lib()
    d = _desc()
    items, rowp = 0x90000, 0xA0000

    def plan(num_items=2, max_slots=3, pt=256, private_parts=0, it=items, rp=rowp,
             private_tokens=0, reserved0=0):
        return pba.SharedPlanDesc(num_items, max_slots, pt, private_parts, it, rp,
                                  private_tokens, reserved0)

    def call(desc, p, ws=0x80000, wsb=1 << 30, batch=2, q=0x30000):
        return lib.pba_paged_decode_shared(ctypes.byref(desc), q, 8, 0x40000, 4, 0x50000, batch,
                                           ctypes.c_float(0.1), 0x60000, NULL,
                                           None if p is None else ctypes.byref(p), ws, wsb, NULL)

    assert call(d, None) == -1
    assert call(_desc(dtype=0), plan()) == -4            # bf16 only
    assert call(d, plan(pt=100)) == -4
    assert call(d, plan(pt=0)) == -4
    assert call(d, plan(private_parts=-1)) == -3
    assert call(d, plan(max_slots=0)) == -3
    assert call(d, plan(num_items=-1)) == -3
    assert call(d, plan(private_tokens=-1)) == -3
    assert call(d, plan(reserved0=1)) == -3
    assert call(d, plan(it=None)) == -1
    assert call(d, plan(rp=None)) == -1
    assert call(d, plan(), batch=70000) == -4
    assert call(d, plan(), batch=0) == 0
    need = lib.pba_paged_decode_shared_workspace_bytes(ctypes.byref(d), 8, 2, 4, ctypes.byref(plan()))
    rows = 2 * 8
    up = lambda x: (x + 255) // 256 * 256
    assert need == up(2 * 2 * 4) + up(rows * 3 * 2 * 4) + rows * 3 * 128 * 4
    assert call(d, plan(), ws=NULL, wsb=0) == -5
    assert call(d, plan(), wsb=need - 1) == -5
    assert lib.pba_paged_decode_shared_workspace_bytes(
        ctypes.byref(d), 8, 2, 4, ctypes.byref(plan(max_slots=1))) == 0
    # Short private ranges (packed four rows per work-group) need the same workspace.
    for ptok in (1, 128, 129):
        assert lib.pba_paged_decode_shared_workspace_bytes(
            ctypes.byref(d), 8, 2, 4, ctypes.byref(plan(private_tokens=ptok))) == need
    assert lib.pba_paged_decode_shared_workspace_bytes(
        ctypes.byref(_desc(dtype=0)), 8, 2, 4, ctypes.byref(plan())) == 0
    assert call(d, plan(), q=0x30008) == -4


def test_kernel_view_host_rules():
    """A kernel view (split_log2 > 0) is for the decode calls only: kv_append
    and block_copy reject it before any launch; expansion and packing reject
    bad sizes."""
    import block_table_attention_amd as pba

    lib = _lib()
    # Tiles of 32 rows (the allocator view's strides) seen as 16-row kernel blocks.
    view = _desc(split_log2=1, num_blocks=8, block_size=16, k_stride_head=32 * 128,
                 v_stride_head=32 * 128, k_stride_block=2 * 32 * 128, v_stride_block=2 * 32 * 128)
    assert lib.pba_kv_append(ctypes.byref(view), 0x30000, 4, 0x40000, 0x50000, NULL) == -4
    assert lib.pba_block_copy(ctypes.byref(view), 0x30000, 0x30010, 4, NULL) == -4
    need = lib.pba_paged_decode_workspace_bytes(ctypes.byref(view), 8, 2, 64, 256)
    assert need > 0
    assert lib.pba_expand_block_tables(0x1000, 4, 5, 0x2000, NULL) == -4
    assert lib.pba_expand_block_tables(0x1000, -1, 1, 0x2000, NULL) == -3
    assert lib.pba_expand_block_tables(NULL, 0, 1, NULL, NULL) == 0
    assert lib.pba_expand_block_tables(NULL, 4, 1, 0x2000, NULL) == -1
    assert lib.pba_pack_block_tables(0x1000, 70000, 4, 0x2000, 0x3000, NULL) == -4
    assert lib.pba_pack_block_tables(0x1000, 2, -1, 0x2000, 0x3000, NULL) == -3
    assert lib.pba_pack_block_tables(NULL, 2, 4, 0x2000, 0x3000, NULL) == -1
    assert lib.pba_paged_decode_ragged(ctypes.byref(view), 0x30000, 8, 0x40000, NULL, 4, 0x50000,
                                       2, ctypes.c_float(0.1), 0x60000, NULL, 0, NULL, 0, NULL) == -1


def test_noalloc_limits_rejected_on_the_host():
    """The allocation-free decode rejects arguments that need more than its
    fixed scratch (states, then counters) and NULL pointers before it looks
    up the scratch or launches anything: no GPU is needed to see it."""
    import block_table_attention_amd as pba

    lib = _lib()
    d = _desc(num_kv_heads=8, k_stride_block=8 * 16 * 128, v_stride_block=8 * 16 * 128)
    ws = lib.pba_paged_decode_workspace_bytes(ctypes.byref(d), 64, 64, 2048, 256)
    assert ws > pba.NOALLOC_STATE_BYTES
    assert lib.pba_paged_decode_noalloc(ctypes.byref(d), 0x30000, 64, 0x40000, 2048, 0x50000, 64,
                                        ctypes.c_float(0.1), 0x60000, NULL, 256, NULL) == -11
    assert 40000 * 8 * 4 > pba.NOALLOC_COUNTER_BYTES
    assert lib.pba_paged_decode_noalloc(ctypes.byref(d), 0x30000, 8, 0x40000, 32, 0x50000, 40000,
                                        ctypes.c_float(0.1), 0x60000, NULL, 256, NULL) == -11
    assert lib.pba_paged_decode_noalloc(ctypes.byref(d), NULL, 8, 0x40000, 64, 0x50000, 4,
                                        ctypes.c_float(0.1), 0x60000, NULL, 256, NULL) == -1
    assert lib.pba_paged_decode_noalloc(NULL, 0x30000, 8, 0x40000, 64, 0x50000, 4,
                                        ctypes.c_float(0.1), 0x60000, NULL, 256, NULL) == -1
    assert pba.STATUS[-11] == "PBA_ERR_SCRATCH_LIMIT"
    assert "scratch" in lib.pba_status_string(-11).decode()


def test_decode_plan_reasons_and_fallbacks():
    """pba_paged_decode_plan_ex reports the decomposition, the partition
    request to pass on, and why -- including why a balanced choice became the
    grid -- from a summary of the lengths (no GPU: 256 CUs assumed)."""
    import block_table_attention_amd as pba

    bf = _desc(num_kv_heads=8, k_stride_block=8 * 16 * 128, v_stride_block=8 * 16 * 128)
    f32 = _desc(dtype=0, num_kv_heads=8, k_stride_block=8 * 16 * 128, v_stride_block=8 * 16 * 128)
    auto = pba.PARTITIONS_AUTO
    ragged = [100] * 127 + [8192]
    p = pba.paged_decode_plan_ex(bf, 32, 128, 512, auto, ragged)
    assert (p["decomposition"], p["partition_request"], p["reason"], p["fallback"]) == \
        ("balanced", -1, "ragged lengths", "none")
    assert p["workspace_bytes"] == _lib().pba_paged_decode_workspace_bytes(ctypes.byref(bf), 32, 128,
                                                                           512, -1) > 0
    p = pba.paged_decode_plan_ex(f32, 32, 128, 512, auto, ragged)
    assert p["decomposition"] == "grid" and p["fallback"] == "fallback: fp32 pool"
    assert p["partition_request"] == 512 and p["partition_tokens"] == 512
    p = pba.paged_decode_plan_ex(bf, 32, 4001, 512, auto, [100] * 4000 + [8192])
    assert p["fallback"] == "fallback: more than 2048 rows" and p["partition_request"] == 512
    p = pba.paged_decode_plan_ex(bf, 128, 128, 512, auto, ragged)        # G = 16 at d = 128
    assert p["fallback"] == "fallback: LDS above 64 KiB" and p["decomposition"] == "grid"
    p = pba.paged_decode_plan_ex(bf, 32, 128, 512, pba.PARTITIONS_BALANCED)
    assert p["decomposition"] == "balanced" and p["reason"] == "requested"
    p = pba.paged_decode_plan_ex(f32, 32, 128, 512, pba.PARTITIONS_BALANCED)
    assert p["decomposition"] == "grid" and p["fallback"] == "fallback: fp32 pool"
    mild = list(range(400, 2400, 12))                                   # 167 rows, longest 2392
    p = pba.paged_decode_plan_ex(bf, 32, len(mild), 150, auto, mild)
    assert p["reason"] == "mildly ragged lengths" and p["partition_request"] == 512
    p = pba.paged_decode_plan_ex(bf, 32, 64, 128, auto, [2000] * 64)
    assert p["reason"] == "uniform lengths" and p["partition_request"] == 0
    p = pba.paged_decode_plan_ex(bf, 32, 8, 1024, auto, [16384] * 8)
    assert p["reason"] == "few rows" and p["num_partitions"] == 4       # 64 pairs, 4 per row
    p = pba.paged_decode_plan_ex(bf, 32, 8, 1024, auto)
    assert p["reason"] == "table width"
    p = pba.paged_decode_plan_ex(bf, 32, 8, 1024, 512)
    assert p["reason"] == "requested" and p["partition_tokens"] == 512
    # The decode calls take the resolved request, never AUTO.
    lib = _lib()
    assert lib.pba_paged_decode(ctypes.byref(bf), 0x30000, 32, 0x40000, 4, 0x50000, 2,
                                ctypes.c_float(0.1), 0x60000, NULL, auto, 0x70000, 1 << 30,
                                NULL) == -3
