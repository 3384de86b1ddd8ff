"""The package's caller-side BlockManager against the oracle allocator.

Both follow the same rules (free FIFO, reference counts, fork, the three append
paths); given the same FIFO start they must produce identical tables, slots,
copy pairs and free lists for any script.  The bench executes workload scripts
with BlockManager, so this pins the bench's inputs to the oracle's.
"""
import copy

import numpy as np
import pytest

import workloads as wl
from block_table_attention_amd.blocks import BlockManager, OutOfBlocks
from oracle.allocator import BlockAllocator, OutOfBlocks as OracleOut


def _state(m: BlockManager, rids):
    return (tuple(m._free), tuple(int(x) for x in m._ref),
            tuple((r, tuple(m.table(r)), m.length(r)) for r in rids))


def _oracle_state(a: BlockAllocator, rids):
    return (tuple(a.free), tuple(a.ref), tuple((r, tuple(a.table(r)), a.length(r)) for r in rids))


def _run_both(w: wl.Workload):
    order = wl.fifo_order(w)
    a = BlockAllocator(w.shape.num_blocks, w.shape.block_size, free_order=order)
    m = BlockManager(w.shape.num_blocks, w.shape.block_size, free_order=order)
    for act in w.actions:
        if act[0] == "new":
            assert a.new_request() == m.new_request()
        elif act[0] in ("prefill", "append"):
            rid = act[1]
            n = act[2] if act[0] == "prefill" else 1
            before = len(a.trace)
            a.prefill(rid, n)
            ops = a.trace[before:]
            slots, copies = m.append(rid, n)
            assert [op[1:] for op in ops if op[0] == "copy"] == copies
            assert [op[3] for op in ops if op[0] == "write"] == slots.tolist()
            # Copies come before the first write of the call.
            if copies:
                assert ops[0][0] == "copy"
        elif act[0] == "fork":
            assert a.fork(act[1]) == m.fork(act[1])
        elif act[0] == "release":
            a.release(act[1])
            m.release(act[1])
    live = sorted(a.tables)
    assert _oracle_state(a, live) == _state(m, live)
    np.testing.assert_array_equal(
        m.block_tables(w.decode),
        np.array([a.table(r) + [-1] * (max(len(a.table(x)) for x in w.decode) - len(a.table(r)))
                  for r in w.decode], dtype=np.int32))
    np.testing.assert_array_equal(m.seq_lens(w.decode), [a.length(r) for r in w.decode])
    return a, m


@pytest.mark.parametrize("make", [
    wl.tiny,
    wl.batch32,
    lambda: wl.shared_prefix(children=16),
    lambda: wl.shared_prefix(prefix=37, children=5, lo=1, hi=40, num_blocks=64),
    lambda: wl.lognormal(16, batch=32),
    lambda: wl.lognormal(256, batch=32),
], ids=["tiny", "batch32", "shared_prefix16", "shared_prefix_small", "lognormal16", "lognormal256"])
def test_workload_scripts_match_oracle(make):
    _run_both(make())


def test_shared_prefix_step_copies():
    """Every sibling's divergent append copies the shared tail exactly when the
    child's length is not a multiple of P (the pages' boundary rule)."""
    w = wl.shared_prefix(children=16)
    _, m = _run_both(w)
    kids = w.decode[:16]
    sibs = w.decode[16:]
    for k, s in zip(kids, sibs):
        tk, ts = m.table(k), m.table(s)
        T = m.length(k)
        assert m.length(s) == T + 1
        if T % 16:
            assert ts[:-1] == tk[:-1] and ts[-1] != tk[-1]
        else:
            assert ts[:-1] == tk and len(ts) == len(tk) + 1


@pytest.mark.parametrize("seed", range(12))
def test_random_scripts(seed):
    """Random new / fork / release / multi-token appends on a tiny pool, with
    out-of-blocks failures that must leave the state unchanged."""
    rng = np.random.default_rng(1000 + seed)
    nb, P = 10, 4
    order = rng.permutation(nb)
    a = BlockAllocator(nb, P, free_order=order)
    m = BlockManager(nb, P, free_order=order)
    live = []
    for _ in range(60):
        op = rng.integers(0, 10)
        if op == 0 or not live:
            assert a.new_request() == m.new_request()
            live.append(m._next_rid - 1)
        elif op == 1:
            r = live[rng.integers(len(live))]
            assert a.fork(r) == m.fork(r)
            live.append(m._next_rid - 1)
        elif op == 2 and len(live) > 1:
            r = live.pop(rng.integers(len(live)))
            a.release(r)
            m.release(r)
        else:
            r = live[rng.integers(len(live))]
            n = int(rng.integers(0, 7))
            snap = _state(m, live)
            try:
                slots, copies = m.append(r, n)
            except OutOfBlocks:
                assert _state(m, live) == snap
                # The oracle runs out too on the same tokens (it may have
                # written some of them first, so it runs on a copy).
                with pytest.raises(OracleOut):
                    copy.deepcopy(a).prefill(r, n)
                continue
            before = len(a.trace)
            a.prefill(r, n)
            ops = a.trace[before:]
            assert [op[1:] for op in ops if op[0] == "copy"] == copies
            assert [op[3] for op in ops if op[0] == "write"] == slots.tolist()
        a.check_invariants()
        assert _oracle_state(a, live) == _state(m, live)


def test_out_of_blocks_is_atomic():
    m = BlockManager(3, 4)
    r = m.new_request()
    m.append(r, 8)                       # two blocks
    c = m.fork(r)
    snap = _state(m, [r, c])
    with pytest.raises(OutOfBlocks):
        m.append(c, 5)                   # 8 -> 13 tokens needs 2 more blocks, 1 free
    assert _state(m, [r, c]) == snap
    slots, copies = m.append(c, 4)       # exactly one fresh block
    assert copies == [] and len(slots) == 4


def test_block_tables_padding():
    m = BlockManager(8, 16)
    a, b = m.new_request(), m.new_request()
    m.append(a, 40)
    m.append(b, 1)
    t = m.block_tables([a, b])
    assert t.shape == (2, 3) and t.dtype == np.int32
    assert (t[1, 1:] == -1).all()
    assert m.block_tables([a, b], width=5).shape == (2, 5)
    with pytest.raises(ValueError):
        m.block_tables([a, b], width=2)


# ---------------------------------------------------------------------------
# BundleManager: several cache groups, all-or-nothing appends
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(4))
def test_bundle_manager_matches_oracle_bundle_allocator(seed):
    """Random scripts over two groups (P 16 and 32 or 64): the caller-side
    BundleManager and the oracle's BundleAllocator give the same tables,
    slots and copies, group by group."""
    from block_table_attention_amd.blocks import BundleManager
    from oracle.bundles import BundleAllocator

    rng = np.random.default_rng(300 + seed)
    Ps = [16, int(rng.choice([32, 64]))]
    NB = [300, 160]
    orders = [rng.permutation(n).tolist() for n in NB]
    m = BundleManager(NB, Ps, free_orders=orders)
    a = BundleAllocator(NB, Ps, free_orders=orders)
    live = []
    for _ in range(80):
        op = rng.integers(4) if live else 0
        if op == 0:
            assert m.new_request() == a.new_request()
            live.append(len(a.tables) and max(a.tables))
        elif op == 1:
            r = live[int(rng.integers(len(live)))]
            assert m.fork(r) == a.fork(r)
            live.append(max(a.tables))
        elif op == 2 and len(live) > 1:
            r = live.pop(int(rng.integers(len(live))))
            m.release(r)
            a.release(r)
        else:
            r = live[int(rng.integers(len(live)))]
            n = int(rng.integers(1, 30))
            n0 = len(a.trace)
            want = [a.append(r) for _ in range(n)]
            slots, copies = m.append(r, n)
            for g in range(2):
                assert slots[g].tolist() == [w[g] for w in want]
                ocopies = [(op[2], op[3]) for op in a.trace[n0:] if op[0] == "copy" and op[1] == g]
                assert copies[g] == ocopies
        for g in range(2):
            for r in live:
                assert m.groups[g].table(r) == a.table(r, g)


def test_bundle_manager_all_or_nothing():
    from block_table_attention_amd.blocks import BundleManager, OutOfBlocks

    m = BundleManager([8, 2], [16, 16])
    r = m.new_request()
    m.append(r, 32)                        # group 1 full
    state = ([list(g._free) for g in m.groups], [g.table(r) for g in m.groups])
    with pytest.raises(OutOfBlocks):
        m.append(r, 1)
    assert ([list(g._free) for g in m.groups], [g.table(r) for g in m.groups]) == state
    assert m.length(r) == 32


def test_partition_suggestion():
    from block_table_attention_amd.blocks import PARTITIONS_BALANCED, suggest_partition_tokens

    uniform = [16384] * 8
    assert suggest_partition_tokens(uniform, 8) == 0                 # 64 units < 256 CUs
    assert suggest_partition_tokens([1000] * 64, 8) == 0             # not ragged
    ragged = [100] * 127 + [8192]
    assert suggest_partition_tokens(ragged, 8) == PARTITIONS_BALANCED
    pt = suggest_partition_tokens(ragged, 8, balanced_ok=False)
    assert pt % 256 == 0 and 512 <= pt < 8192
    assert suggest_partition_tokens([100] * 4000 + [8192], 8) > 0    # too many rows to balance
    # Mildly ragged batches over half the CUs: 512-token partitions (1024 from
    # 4096 tokens on); under half the CUs, short or uniform: the library plan.
    mild = list(range(101, 2029, 48))                                # 41 rows, 101..2021
    assert suggest_partition_tokens(mild, 4) == 512                  # 164 units > 128
    assert suggest_partition_tokens(mild[:30], 4) == 0               # 120 units < 128
    assert suggest_partition_tokens([x * 4 for x in mild], 8) == 1024
    assert suggest_partition_tokens([x // 2 for x in mild], 8) == 0  # longest < 1536
    assert suggest_partition_tokens([2000] * 40, 8) == 0             # uniform
