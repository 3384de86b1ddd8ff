"""Pins for oracle.bundles: cache groups with a layer axis, whole-bundle
appends and copies, and the all-or-nothing bundle allocator.

* Row and bundle bytes of the pages' two-group fixture, read off the pools'
  own array sizes (0x03B, 0x04E).
* The pages' checked address (0x03F): a row appended at slot 96 of a pool laid
  out in the pages' g1 axis order lands at element 49,285.
* The boundary crossing of 0x03H: offset 0 in both groups, slot ids 0 and 64.
* The two-group copy-on-write trace of 0x05B, and the pool contents it leaves.
* Rollback (0x04F): a failure injected between the groups' reservations, or a
  group that runs out of blocks, leaves the committed state digest unchanged,
  where independent per-group allocators would have moved group 0.
* Group-specific block sizes: each group of the bundle allocator behaves as
  the pinned single-group allocator run on the same operations.
* Layer-major and block-major manifests hold the same rows, and every layer
  of a layered pool equals a single-layer pool replayed with that layer's rows.
* Half bundles are rejected before any group changes.
"""

import numpy as np
import pytest

from oracle import attention as att
from oracle import bundles as bd
from oracle.allocator import BlockAllocator, OutOfBlocks
from oracle.pool import replay


def manifests(P0=16, P1=16, nb0=8, nb1=8, layers=(24, 8), H=4, d=128, dtype="bf16",
              order="layer"):
    k = bd.LAYER_MAJOR_K if order == "layer" else bd.BLOCK_MAJOR_K
    v = bd.LAYER_MAJOR_V if order == "layer" else bd.BLOCK_MAJOR_V
    return [bd.GroupManifest(layers[0], nb0, P0, H, d, dtype, k, v),
            bd.GroupManifest(layers[1], nb1, P1, H, d, dtype, k, v)]


def empty_pool(m, fill=0):
    n = m.elements()
    return bd.LayeredPool(m, np.full(n, fill, dtype=np.uint16), np.full(n, fill, dtype=np.uint16))


def test_row_and_bundle_bytes(golden):
    fx = golden("address_trace.json")["row_bytes"]
    ms = manifests(layers=(fx["g0_layers"], fx["g1_layers"]), H=fx["kv_heads"], d=fx["head_dim"])
    pools = [empty_pool(m) for m in ms]
    # From the arrays themselves: bytes of K and V over all slots of the group.
    for p, want in zip(pools, (fx["g0_row"], fx["g1_row"])):
        total = p.k.nbytes + p.v.nbytes
        assert total // (p.m.num_blocks * p.m.block_size) == want == bd.row_bytes(p.m)
    assert bd.row_bytes(ms[0]) + bd.row_bytes(ms[1]) == fx["rank_row"]
    assert bd.bundle_bytes(ms) == fx["bundle_block_bytes"] == 1 << 20


def test_pages_checked_address(golden):
    """Pool in the pages' g1 axis order [layer, slot, token, head, dim] with
    shape [8, 8, 16, 4, 128]: the row written at slot 96 (block 6, offset 0)
    puts layer 0, head 1, dim 5 at element 49,285, byte 98,570."""
    fx = golden("address_trace.json")["checked_address"]
    L, NB, P, H, d = fx["group"]["shape"]
    axes = ("layer", "block", "token", "head", "dim")
    m = bd.GroupManifest(L, NB, P, H, d, "bf16", axes, axes)
    assert list(row_major_strides_of(m)) == fx["expect"]["strides"]
    pool = empty_pool(m)
    k = np.zeros((1, L, H, d), dtype=np.uint16)
    k[0, 0, 1, 5] = 0x7777
    pool.kv_append([fx["expect"]["slot_id"]], k, np.zeros_like(k))
    hit = np.flatnonzero(pool.k)
    assert hit.tolist() == [fx["expect"]["element_offset"]]
    assert hit[0] * fx["group"]["scalar_bytes"] == fx["expect"]["byte_offset"]


def row_major_strides_of(m):
    s = m.strides("K")
    return [s[a] for a in m.k_axes]


def test_boundary_crossing_two_groups(golden):
    fx = golden("address_trace.json")["boundary_crossing"]
    P = fx["block_size"]
    # Free orders arranged so that the block after C's first one is physical
    # slot 0 in group 0 and slot 4 in group 1, as on the page.
    a = bd.BundleAllocator([8, 8], [P, P], free_orders=[[5, 0, 1, 2, 3, 4, 6, 7],
                                                        [5, 4, 0, 1, 2, 3, 6, 7]])
    C = a.new_request()
    a.prefill(C, fx["token"])
    slots = a.append(C)
    assert [s % P for s in slots] == [fx["offset"], fx["offset"]]
    assert [a.table(C, g)[fx["logical_block"]] for g in (0, 1)] == [fx["g0_physical_slot"],
                                                                    fx["g1_physical_slot"]]
    assert slots == [fx["g0_slot_id"], fx["g1_slot_id"]]


def test_two_group_cow_trace(golden):
    fx = golden("cow_trace.json")["trace"]
    P = fx["P"]
    ms = manifests(nb0=16, nb1=16, layers=(3, 2), H=2, d=64)
    a = bd.BundleAllocator([16, 16], [P, P])
    A = a.new_request()
    a.prefill(A, fx["A_context_before"])
    assert a.lengths[A] % P == fx["A_tail_rows_before"]
    slots = a.append(A)
    assert [s % P for s in slots] == [fx["A_write_offset"]] * 2
    assert not [op for op in a.trace if op[0] == "copy"]
    D = a.fork(A)
    old = [a.table(A, g)[-1] for g in (0, 1)]
    assert all(a.ref[g][old[g]] == fx["shared_tail_refs_after_fork"] for g in (0, 1))
    n0 = len(a.trace)
    slots = a.append(D)
    new_ops = a.trace[n0:]
    # Both groups copy their tail, then both write offset 2 of the copy.
    copies = [op for op in new_ops if op[0] == "copy"]
    writes = [op for op in new_ops if op[0] == "write"]
    assert [op[1] for op in copies] == [0, 1] and [op[2] for op in copies] == old
    assert new_ops[:2] == copies and len(writes) == 2
    assert [s % P for s in slots] == [fx["D_write_offset"]] * 2
    for g in (0, 1):
        assert a.ref[g][old[g]] == fx["old_tail_refs_after"]
        assert a.ref[g][a.table(D, g)[-1]] == fx["new_tail_refs"]
        assert a.table(D, g)[:-1] == a.table(A, g)[:-1]
    assert a.lengths[D] == fx["D_context_after"]
    a.check_invariants()
    # Replay into layered pools: D sees A's rows [0, 34) and its own row 34.
    rng = np.random.default_rng(3)
    n_w = sum(1 for op in a.trace if op[0] == "write") // 2
    rows = [(rng.integers(0, 1 << 16, size=(n_w, m.layers, m.kv_heads, m.head_dim), dtype=np.uint16),
             rng.integers(0, 1 << 16, size=(n_w, m.layers, m.kv_heads, m.head_dim), dtype=np.uint16))
            for m in ms]
    pools = [empty_pool(m) for m in ms]
    bd.replay_bundle_trace(pools, a.trace, [r[0] for r in rows], [r[1] for r in rows])
    for g, p in enumerate(pools):
        for layer in range(p.m.layers):
            lp = p.layer_pool(layer)
            KA, _ = lp.gather(a.table(A, g), 34, 1)
            KD, _ = lp.gather(a.table(D, g), 35, 1)
            assert np.array_equal(KD[:34], KA, equal_nan=True)


def _setup_crossing():
    a = bd.BundleAllocator([6, 6], [16, 16], free_orders=[[3, 1, 4, 0, 5, 2], [2, 5, 0, 4, 1, 3]])
    r = a.new_request()
    a.prefill(r, 16)                      # the next append crosses into block 1 of both groups
    return a, r


def test_rollback_restores_predecessor(golden):
    fx = golden("bundle_rollback.json")
    a, r = _setup_crossing()
    before = a.state_digest()
    n_trace = len(a.trace)
    with pytest.raises(bd.InjectedFailure):
        a.append(r, fail_at_group=fx["failing_group"])
    assert fx["published"] is False and len(a.trace) == n_trace
    assert (a.state_digest() == before) is fx["predecessor_digest_restored"]
    # Returning the reserved block to the tail instead of the head would not
    # restore the digest: the FIFO order is part of the committed state.
    b = bd.BundleAllocator([6, 6], [16, 16], free_orders=[[3, 1, 4, 0, 5, 2], [2, 5, 0, 4, 1, 3]])
    rb = b.new_request()
    b.prefill(rb, 16)
    blk = b.free[0].popleft()
    b.free[0].append(blk)
    assert b.state_digest() != before
    # After the failure the same append succeeds and both groups move.
    slots = a.append(r)
    assert [len(a.table(r, g)) for g in (0, 1)] == [2, 2] and all(s % 16 == 0 for s in slots)
    a.check_invariants()


def test_out_of_blocks_in_one_group_moves_no_group():
    a = bd.BundleAllocator([6, 2], [16, 16])
    r = a.new_request()
    a.prefill(r, 32)                      # group 1 is now full (2 blocks)
    before = a.state_digest()
    with pytest.raises(OutOfBlocks):
        a.append(r)
    assert a.state_digest() == before
    # Two independent single-group allocators would have moved group 0.
    g0, g1 = BlockAllocator(6, 16), BlockAllocator(2, 16)
    r0, r1 = g0.new_request(), g1.new_request()
    g0.prefill(r0, 32)
    g1.prefill(r1, 32)
    g0.append(r0)
    with pytest.raises(OutOfBlocks):
        g1.append(r1)
    assert len(g0.table(r0)) == 3 and len(g1.table(r1)) == 2


@pytest.mark.parametrize("seed", range(6))
def test_group_specific_block_sizes_match_single_group_allocator(seed):
    """Each group of the bundle allocator (P_0 = 16, P_1 = 32 or 64) behaves
    exactly as the single-group allocator with that group's P and free order
    on the same operations: tables, slots, copies, refcounts."""
    rng = np.random.default_rng(40 + seed)
    Ps = [16, int(rng.choice([32, 64]))]
    NB = [400, 200]
    orders = [rng.permutation(n).tolist() for n in NB]
    a = bd.BundleAllocator(NB, Ps, free_orders=orders)
    singles = [BlockAllocator(NB[g], Ps[g], free_order=orders[g]) for g in range(2)]
    live = []
    for step in range(120):
        op = rng.integers(4) if live else 0
        if op == 0:
            r = a.new_request()
            for s in singles:
                assert s.new_request() == r
            live.append(r)
        elif op == 1:
            r = live[int(rng.integers(len(live)))]
            c = a.fork(r)
            for s in singles:
                assert s.fork(r) == c
            live.append(c)
        elif op == 2 and len(live) > 1:
            r = live.pop(int(rng.integers(len(live))))
            a.release(r)
            for s in singles:
                s.release(r)
        else:
            r = live[int(rng.integers(len(live)))]
            for _ in range(int(rng.integers(1, 40))):
                slots = a.append(r)
                for g, s in enumerate(singles):
                    assert s.append(r) == slots[g]
        for g, s in enumerate(singles):
            assert a.ref[g] == s.ref and list(a.free[g]) == list(s.free)
            for r in live:
                assert a.table(r, g) == s.table(r)
    a.check_invariants()
    # Copies per group are the single allocators' copies, in the same order.
    for g, s in enumerate(singles):
        mine = [(op[2], op[3]) for op in a.trace if op[0] == "copy" and op[1] == g]
        theirs = [(op[1], op[2]) for op in s.trace if op[0] == "copy"]
        assert mine == theirs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layer_and_block_major_pools_agree_with_single_layer_pools(dtype):
    rng = np.random.default_rng(11)
    P, NB, H, d, L = 16, 12, 2, 64, 3
    bits = np.uint16 if dtype == "bf16" else np.uint32
    top = 1 << (16 if dtype == "bf16" else 32)
    a = bd.BundleAllocator([NB], [P], free_orders=[rng.permutation(NB).tolist()])
    r0 = a.new_request()
    a.prefill(r0, 37)
    r1 = a.fork(r0)
    a.prefill(r1, 9)                      # copy-on-write of the 5-row tail
    a.prefill(r0, 20)
    n_w = sum(1 for op in a.trace if op[0] == "write")
    k = rng.integers(0, top, size=(n_w, L, H, d), dtype=np.uint64).astype(bits)
    v = rng.integers(0, top, size=(n_w, L, H, d), dtype=np.uint64).astype(bits)
    init = rng.integers(0, top, size=NB * L * H * P * d, dtype=np.uint64).astype(bits)
    pools = {}
    for order in ("layer", "block"):
        kx = bd.LAYER_MAJOR_K if order == "layer" else bd.BLOCK_MAJOR_K
        vx = bd.LAYER_MAJOR_V if order == "layer" else bd.BLOCK_MAJOR_V
        m = bd.GroupManifest(L, NB, P, H, d, dtype, kx, vx)
        p = bd.LayeredPool(m, init, init)
        bd.replay_bundle_trace([p], a.trace, [k], [v])
        pools[order] = p
    single_trace = [("copy", op[2], op[3]) if op[0] == "copy" else ("write", op[2], op[3], op[4])
                    for op in a.trace]
    for layer in range(L):
        # A single-layer pool starting from the layer-major pool's initial bits.
        m = pools["layer"].m
        start = bd.LayeredPool(m, init, init).layer_pool(layer)
        replay(start, single_trace, k[:, layer], v[:, layer])
        for order in ("layer", "block"):
            lp = pools[order].layer_pool(layer)
            for r, T in ((r0, 57), (r1, 46)):
                for h in range(H):
                    K1, V1 = lp.gather(a.table(r, 0), T, h)
                    K2, V2 = start.gather(a.table(r, 0), T, h)
                    assert np.array_equal(K1, K2, equal_nan=True)
                    assert np.array_equal(V1, V2, equal_nan=True)
    # The two manifests hold different memory orders of the same rows.
    assert pools["layer"].digest() != pools["block"].digest()


def test_half_bundles_rejected():
    ms = manifests(nb0=4, nb1=4, layers=(2, 1), H=1, d=64)
    pools = [empty_pool(m) for m in ms]
    before = [p.digest() for p in pools]
    rows = [np.ones((2, m.layers, 1, 64), dtype=np.uint16) for m in ms]
    with pytest.raises(bd.HalfBundle):
        bd.bundle_append(pools, [[0, 17], [0, -1]], rows, rows)   # token 1 in group 0 only
    with pytest.raises(bd.HalfBundle):
        bd.bundle_append(pools, [[0, 17]], rows[:1], rows[:1])    # group 1 missing
    with pytest.raises(ValueError):                              # bad pair in group 1
        bd.bundle_copy(pools, [[(0, 1)], [(2, 2)]])
    assert [p.digest() for p in pools] == before
    bd.bundle_append(pools, [[0, 17], [3, -1 + 5]], rows, rows)
    bd.bundle_copy(pools, [[(0, 1)], []])                        # groups may copy unequal counts
    assert [p.digest() for p in pools] != before
    # A trace whose token is written to one group only.
    with pytest.raises(bd.HalfBundle):
        bd.replay_bundle_trace(pools, [("write", 0, 0, 0, 5), ("write", 0, 0, 1, 6)],
                               [r for r in rows], [r for r in rows])


def test_layer_decode_through_layered_pool():
    """Decode of one layer through ``layer_pool`` equals attention over the
    rows that were appended for that layer (plain softmax, binary64)."""
    rng = np.random.default_rng(5)
    m = bd.GroupManifest(2, 8, 16, 2, 64, "f32", bd.BLOCK_MAJOR_K, bd.BLOCK_MAJOR_V)
    a = bd.BundleAllocator([8], [16], free_orders=[rng.permutation(8).tolist()])
    r = a.new_request()
    a.prefill(r, 40)
    vals = rng.standard_normal((40, 2, 2, 64)).astype(np.float32)
    valv = rng.standard_normal((40, 2, 2, 64)).astype(np.float32)
    p = bd.LayeredPool(m, np.zeros(m.elements(), np.uint32), np.zeros(m.elements(), np.uint32))
    bd.replay_bundle_trace([p], a.trace, [vals.view(np.uint32)], [valv.view(np.uint32)])
    q = rng.standard_normal((1, 4, 64)).astype(np.float32)
    for layer in range(2):
        out, _ = att.paged_decode(p.layer_pool(layer), q.view(np.uint32), [a.table(r, 0)],
                                  np.array([40]), 0.125)
        for h in range(4):
            kv = h // 2
            s = (vals[:, layer, kv].astype(np.float64) @ q[0, h].astype(np.float64)) * 0.125
            w = np.exp(s - s.max())
            ref = (w / w.sum()) @ valv[:, layer, kv].astype(np.float64)
            assert np.max(np.abs(out[0, h] - ref)) <= 1e-12
