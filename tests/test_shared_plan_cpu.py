"""The caller-side shared-prefix plan (blocks.shared_plan) on the CPU.

* Contract, by brute force: for every row the chunk-first pieces covering it
  and its private pieces tile [0, T) exactly, its slots are 0 .. n-1, and every
  row an item covers maps the item's blocks to the same ids as the item's
  first row.
* Ledger: the plan reads each visible physical row once per work item over
  it -- a chunk once per 64 query columns, a private row once (the pages'
  physical-versus-logical K/V count of 0x0BE, at the kernel's group size).
* Semantics: evaluating the plan's slots with the oracle's partial states and
  merging them in slot order equals monolithic attention (oracle) to binary64
  rounding.
"""
import math

import numpy as np
import pytest

import bench
import workloads as wl
from block_table_attention_amd.blocks import BlockManager, shared_chunks, shared_plan, sharing_order
from harness import execute, oracle_pool
from oracle import attention as att
from oracle.bits import bits_to_f64


def _pieces(plan, lens):
    """Per row: list of (tb, te, slot) from items and private pieces."""
    B = len(lens)
    per = [[] for _ in range(B)]
    for row0, nrows, tb, te, slot, tiles, _, _ in plan.items.tolist():
        for r in range(row0, row0 + nrows):
            per[r].append((tb, te, slot))
    for r in range(B):
        pb, ps = plan.row_private[r]
        k = 0
        for t in range(int(pb), int(lens[r]), plan.partition_tokens):
            per[r].append((t, min(int(lens[r]), t + plan.partition_tokens), int(ps) + k))
            k += 1
    return per


def check_contract(plan, tables, lens, P, G):
    rpt = 16 // G
    align = min(P, 32)
    for row0, nrows, tb, te, slot, tiles, z0, z1 in plan.items.tolist():
        assert z0 == 0 and z1 == 0 and tb % align == 0 and tb < te
        assert tiles in (1, 2, 4) and 1 <= nrows <= tiles * rpt
        for r in range(row0, row0 + nrows):
            assert te <= lens[r]
            j0, j1 = tb // P, -(-te // P)
            assert (tables[r, j0:j1] == tables[row0, j0:j1]).all()
    for r, pcs in enumerate(_pieces(plan, lens)):
        pcs.sort()
        at = 0
        for tb, te, _ in pcs:
            assert tb == at
            at = te
        assert at == lens[r]
        slots = sorted(p[2] for p in pcs)
        assert slots == list(range(len(slots))) and len(slots) <= plan.max_slots
        assert plan.row_private[r, 0] % align == 0
        assert lens[r] - plan.row_private[r, 0] <= plan.private_tokens
    # The bound is tight (at least one position: a plan with no private
    # position still gives a nonzero bound).
    assert plan.private_tokens == max(1, int(max(lens - plan.row_private[:, 0])))


def plan_kv_rows(plan, lens):
    """K/V rows the plan reads: each item once (a tiled item's four tiles share
    one read), each private piece once."""
    rows = sum(te - tb for _, _, tb, te, _, _, _, _ in plan.items.tolist())
    rows += sum(max(0, int(lens[r]) - int(plan.row_private[r, 0])) for r in range(len(lens)))
    return rows


def _ordered(w):
    p = bench.plan_script(w)
    order = sharing_order(p.tables)
    return p.tables[order], p.seq_lens[order], order


@pytest.mark.parametrize("pt", [256, 512, 2048])
def test_shared_prefix_workload_plan(pt):
    w = wl.shared_prefix()
    tables, lens, _ = _ordered(w)
    P, G = w.shape.block_size, w.shape.num_q_heads // w.shape.num_kv_heads
    plan = shared_plan(tables, lens, P, G, pt)
    check_contract(plan, tables, lens, P, G)
    # The root chunk is the 2000-token prefix over all 128 rows.
    assert plan.chunks[0] == (0, 128, 0, 2000)
    unique = np.unique(bench.visible_slots(tables, lens, P)).size
    # Every visible physical row is read once per item over it: a chunk once
    # per group of 64 query columns (16 rows at G = 4), private rows once.
    extra = sum((t1 - t0) * (_items_per_piece(b - a, G) - 1) for a, b, t0, t1 in plan.chunks)
    assert plan_kv_rows(plan, lens) == unique + extra
    # The prefix: 8 reads for 128 rows instead of 128.
    assert _items_per_piece(128, G) == 8
    logical = int(lens.sum())
    assert plan_kv_rows(plan, lens) * 7 < logical     # 303,270 logical rows, 40,182 read


def _items_per_piece(rows, G, per_item=4):
    tiles = -(-rows // (16 // G))
    n = 0
    while tiles > 0:
        t = min(per_item, 4 if tiles >= 4 else (2 if tiles >= 2 else 1))
        tiles -= t
        n += 1
    return n


def test_no_sharing_is_all_private():
    w = wl.lognormal(16, batch=32)
    tables, lens, _ = _ordered(w)
    plan = shared_plan(tables, lens, 16, 4, 256)
    assert plan.items.shape == (0, 8) and plan.chunks == []
    assert (plan.row_private[:, 0] == 0).all() and (plan.row_private[:, 1] == 0).all()
    check_contract(plan, tables, lens, 16, 4)


def test_page_tree_from_block_tables():
    """The pages' four-sequence tree (0x0BB) realised with blocks of P = 16:
    C0 2 blocks over all, C1 1 block over {0, 1}, C2 2 blocks over {2, 3},
    then private leaves; threshold 1 yields exactly C0, C1, C2."""
    m = BlockManager(64, 16)
    root = m.new_request()
    m.append(root, 32)
    left, right = m.fork(root), m.fork(root)
    m.append(left, 16)
    m.append(right, 32)
    s0, s1 = m.fork(left), m.fork(left)
    s2, s3 = m.fork(right), m.fork(right)
    for r, n in [(s0, 32), (s1, 16), (s2, 16), (s3, 16)]:
        m.append(r, n)
    rows = [s0, s1, s2, s3]
    tables = m.block_tables(rows)
    lens = m.seq_lens(rows)
    chunks, private = shared_chunks(tables, lens, 16, threshold=1)
    assert chunks == [(0, 4, 0, 32), (0, 2, 32, 48), (2, 4, 32, 64)]
    assert private.tolist() == [48, 48, 64, 64]
    plan = shared_plan(tables, lens, 16, 1, 256)
    check_contract(plan, tables, lens, 16, 1)
    assert plan.private_tokens == 32  # s0's 32 private rows; the others have 16
    # Logical pairs 19, unique 10 (in blocks here: 19 and 10 blocks of 16 rows).
    assert int(lens.sum()) // 16 == 19
    assert plan_kv_rows(plan, lens) // 16 == 10


@pytest.mark.parametrize("seed", range(4))
def test_random_fork_trees(seed):
    """Random fork trees with partial tails: the contract holds for every
    threshold, and threshold 1 reads each visible physical row once."""
    rng = np.random.default_rng(500 + seed)
    P = int(rng.choice([16, 32, 64]))
    m = BlockManager(4096, P, free_order=rng.permutation(4096))
    live = [m.new_request()]
    m.append(live[0], int(rng.integers(1, 300)))
    for _ in range(25):
        r = live[int(rng.integers(len(live)))]
        c = m.fork(r)
        m.append(c, int(rng.integers(1, 200)))
        live.append(c)
    tables = m.block_tables(live)
    lens = m.seq_lens(live)
    order = sharing_order(tables)
    tables, lens = tables[order], lens[order]
    for G, thr in [(4, 1), (1, 1), (8, 0), (2, 3)]:
        plan = shared_plan(tables, lens, P, G, 256, threshold=thr)
        check_contract(plan, tables, lens, P, G)
    plan = shared_plan(tables, lens, P, 4, 256, threshold=1)
    unique = np.unique(bench.visible_slots(tables, lens, P)).size
    # Rows a single sequence owns are private; a partial block two rows share
    # can only be read per row (it is not whole), so the plan may read a few
    # rows twice but never fewer than the unique ones.
    assert plan_kv_rows(plan, lens) >= unique


def test_plan_slots_merge_to_monolithic():
    """Evaluate every slot of a small shared-prefix plan with the oracle's
    partial states and merge them in slot order: equal to the oracle's
    monolithic decode to 1e-13."""
    w = wl.shared_prefix(children=6, prefix=300, lo=3, hi=90, num_blocks=200)
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    order = sharing_order(ex.tables)
    tables, lens = ex.tables[order], ex.seq_lens[order]
    qb = wl.q_bits(w)[order]
    P, Hkv = w.shape.block_size, w.shape.num_kv_heads
    G = w.shape.num_q_heads // Hkv
    plan = shared_plan(tables, lens, P, G, 256)
    check_contract(plan, tables, lens, P, G)
    assert len(plan.chunks) > 1
    scale = 1 / math.sqrt(w.shape.head_dim)
    ref, ref_lse = att.paged_decode(opool, qb, list(tables), lens, scale)
    q = bits_to_f64(qb, w.shape.dtype)
    per = _pieces(plan, lens)
    for r in range(len(lens)):
        for h in range(Hkv):
            K, V = opool.gather(tables[r], int(lens[r]), h)
            states = [None] * len(per[r])
            for tb, te, slot in per[r]:
                states[slot] = att.partial_state(q[r, h * G:(h + 1) * G], K[tb:te], V[tb:te], scale)
            O, L = att.merge_states(states)
            assert np.max(np.abs(O - ref[r, h * G:(h + 1) * G])) <= 1e-13
            assert np.max(np.abs(L - ref_lse[r, h * G:(h + 1) * G])) <= 1e-13


# ---------------------------------------------------------------------------
# The library's planner (pba_shared_plan_build) through ctypes, pinned to the
# oracle's shared-execution ledgers on the pages' four-sequence tree.
# ---------------------------------------------------------------------------
def _fixture_tables(golden):
    """The pages' chunk tree (0x0BB) as block tables with one 16-token block
    per fixture row: chunk c of n rows gets n consecutive block ids, and each
    sequence's table is its path's blocks in order."""
    t = golden("shared_execution.json")["tree"]
    ids, nxt = {}, 0
    for name in sorted(t["chunks"]):
        n = t["chunks"][name][0]
        ids[name] = list(range(nxt, nxt + n))
        nxt += n
    rows = [[b for c in path for b in ids[c]] for path in t["paths"]]
    width = max(len(r) for r in rows)
    tables = np.full((len(rows), width), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    lens = np.array([16 * len(r) for r in rows], dtype=np.int32)
    tree = [(t["chunks"][c][0], tuple(t["chunks"][c][1])) for c in sorted(t["chunks"])]
    return tables, lens, tree, t["expect"]


@pytest.mark.parametrize("threshold", [0, 1, 2, 3, 4])
def test_library_planner_matches_oracle_ledgers(golden, threshold):
    """Chunk-first partial rows and K/V rows read by the library's plan equal
    the oracle's ChunkAttention ledgers (in 16-token blocks) at every
    threshold; threshold 1 gives the pages' 8 partial rows and 10 unique rows
    out of 19 logical ones."""
    import ctypes
    import block_table_attention_amd as pba
    from oracle import shared as S

    tables, lens, tree, expect = _fixture_tables(golden)
    snap = S.random_snapshot(np.random.default_rng(3), tree, G=1, d_qk=2, d_v=3)
    res = S.chunk_attention(snap, 1.0, threshold)
    B, width = tables.shape
    params = pba.SharedPlanParams(16, 1, 256, threshold, 1, 0)
    info = pba.SharedPlanInfo()
    order = np.zeros(B, np.int64)
    priv = np.zeros((B, 2), np.int32)
    st = pba._lib.pba_shared_plan_build(tables.ctypes.data, width, lens.ctypes.data, B,
                                        ctypes.byref(params), order.ctypes.data, None, 0,
                                        priv.ctypes.data, None, 0, ctypes.byref(info))
    assert st == 0
    assert np.array_equal(order, np.arange(B))      # the fixture's rows are already in order
    assert int(lens.sum()) // 16 == expect["logical_pairs"] == 19
    assert info.chunk_rows == res.partial_rows
    assert info.kv_rows_read == 16 * res.kv_rows_read
    if threshold == 1:
        assert info.chunk_rows == expect["partial_rows"] == 8
        assert info.kv_rows_read // 16 == expect["unique_rows"] == 10
        items = np.zeros((info.num_items, 8), np.int32)
        chunks = np.zeros((info.num_chunks, 4), np.int32)
        st = pba._lib.pba_shared_plan_build(tables.ctypes.data, width, lens.ctypes.data, B,
                                            ctypes.byref(params), order.ctypes.data,
                                            items.ctypes.data, info.num_items, priv.ctypes.data,
                                            chunks.ctypes.data, info.num_chunks,
                                            ctypes.byref(info))
        assert st == 0
        assert chunks.tolist() == [[0, 4, 0, 32], [0, 2, 32, 48], [2, 4, 32, 64]]
        assert priv[:, 0].tolist() == [48, 48, 64, 64]
        # Slots: C0, then C1 or C2, then the private range.
        assert priv[:, 1].tolist() == [2, 2, 2, 2] and info.max_slots == 3


def test_library_planner_sizes_and_rejects():
    """A short item buffer returns PBA_ERR_WORKSPACE_TOO_SMALL with the needed
    count and writes nothing; bad parameters are rejected."""
    import ctypes
    import block_table_attention_amd as pba

    m = BlockManager(64, 16)
    root = m.new_request()
    m.append(root, 64)
    kids = [m.fork(root) for _ in range(3)]
    for k in kids:
        m.append(k, 20)
    tables = m.block_tables(kids).astype(np.int32)
    lens = m.seq_lens(kids).astype(np.int32)
    B, width = tables.shape
    info = pba.SharedPlanInfo()
    order = np.full(B, -7, np.int64)
    priv = np.full((B, 2), -7, np.int32)
    items = np.full((1, 8), -7, np.int32)

    def call(params, cap=0, items_ptr=None):
        return pba._lib.pba_shared_plan_build(tables.ctypes.data, width, lens.ctypes.data, B,
                                              ctypes.byref(params), order.ctypes.data, items_ptr,
                                              cap, priv.ctypes.data, None, 0, ctypes.byref(info))

    good = pba.SharedPlanParams(16, 4, 256, 1, 2, 0)
    assert call(good) == 0 and info.num_items == 1 and info.num_chunks == 1
    bigger = pba.SharedPlanParams(16, 4, 256, 0, 1, 0)     # threshold 0: the private runs too
    assert call(bigger, 1, items.ctypes.data) == -5 and info.num_items > 1
    assert (items == -7).all()
    for bad, status in ((pba.SharedPlanParams(24, 4, 256, 1, 2, 0), -4),
                        (pba.SharedPlanParams(16, 4, 300, 1, 2, 0), -4),
                        (pba.SharedPlanParams(16, 4, 256, 1, 3, 0), -4),
                        (pba.SharedPlanParams(16, 32, 256, 1, 2, 0), -4),
                        (pba.SharedPlanParams(16, 4, 256, -1, 2, 0), -3),
                        (pba.SharedPlanParams(16, 4, 256, 1, 2, 5), -3)):
        assert call(bad) == status
