"""Pins for oracle.allocator: worked values, invariants and brute force."""
import copy

import numpy as np
import pytest

from oracle.allocator import AllocatorError, BlockAllocator, OutOfBlocks
from oracle.pool import BitPool, replay


def test_35_tokens_in_16_token_blocks(golden):
    fx = golden("p3_examples.json")["tokens35"]
    a = BlockAllocator(32, fx["P"], free_order=list(range(31, -1, -1)))
    r = a.new_request()
    slots = a.prefill(r, fx["T"])
    t = a.table(r)
    assert len(t) == fx["blocks"] == 3
    assert a.length(r) % fx["P"] == fx["tail_rows"] == 3
    # Free FIFO order: the first three pops of the given order.
    assert t == [31, 30, 29]
    # Every row lands at slot = table[t // P] * P + t % P.
    assert slots == [t[i // 16] * 16 + i % 16 for i in range(35)]
    assert a.n_free() == 29
    a.check_invariants()


def test_fork_shares_and_cow_trace(golden):
    fx = golden("cow_trace.json")["trace"]
    P = fx["P"]
    a = BlockAllocator(16, P)
    A = a.new_request()
    a.prefill(A, fx["A_context_before"])                       # 33 tokens: tail has 1 row
    assert a.length(A) % P == fx["A_tail_rows_before"]
    slot = a.append(A)                                         # private append at token 33
    assert slot % P == fx["A_write_offset"]
    assert a.length(A) == fx["A_context_after"] and a.length(A) % P == fx["A_tail_rows_after"]
    assert not [op for op in a.trace if op[0] == "copy"]
    D = a.fork(A)
    tail = a.table(A)[-1]
    assert all(a.ref[b] == fx["shared_tail_refs_after_fork"] for b in a.table(A))
    n_trace = len(a.trace)
    slot = a.append(D)                                         # divergent append at token 34
    new_ops = a.trace[n_trace:]
    assert new_ops[0][0] == "copy" and new_ops[0][1] == tail
    dst = new_ops[0][2]
    assert new_ops[1] == ("write", D, fx["D_append_token"], dst * P + fx["D_write_offset"])
    assert a.table(D)[-1] == dst and a.table(A)[-1] == tail
    assert a.ref[tail] == fx["old_tail_refs_after"] and a.ref[dst] == fx["new_tail_refs"]
    assert a.length(D) == fx["D_context_after"]
    # The original owner keeps the old tail and appends in place afterwards.
    n_trace = len(a.trace)
    a.append(A)
    assert [op[0] for op in a.trace[n_trace:]] == ["write"]
    a.check_invariants()


def test_boundary_prefix_needs_no_copy(golden):
    fx = golden("cow_trace.json")["shared20"]
    for P, r in [(fx["P"], fx["r"]), (fx["boundary_P"], fx["boundary_r"])]:
        a = BlockAllocator(64, P)
        A = a.new_request()
        a.prefill(A, fx["shared_tokens"])
        B = a.fork(A)
        n = len(a.trace)
        a.append(B)
        copies = [op for op in a.trace[n:] if op[0] == "copy"]
        assert (len(copies) == 1) == (r > 0)
        a.check_invariants()


def test_out_of_blocks_preserves_state():
    a = BlockAllocator(2, 4)
    r = a.new_request()
    a.prefill(r, 8)
    before = a.state_key()
    with pytest.raises(OutOfBlocks):
        a.append(r)
    assert a.state_key() == before
    # COW path: a fork of a partial tail with no free block left.
    a2 = BlockAllocator(2, 4)
    r = a2.new_request()
    a2.prefill(r, 5)
    c = a2.fork(r)
    before = a2.state_key()
    with pytest.raises(OutOfBlocks):
        a2.append(c)
    assert a2.state_key() == before
    a2.check_invariants()


def test_release_returns_blocks_to_fifo_tail():
    a = BlockAllocator(4, 2, free_order=[2, 0, 3, 1])
    r = a.new_request()
    a.prefill(r, 3)                      # takes 2, 0
    assert list(a.free) == [3, 1]
    a.release(r)                         # decref in table order
    assert list(a.free) == [3, 1, 2, 0]
    with pytest.raises(AllocatorError):
        a._decref(2)                     # double release is an error
    a.check_invariants()


def test_parent_release_after_forks_keeps_prefix():
    a = BlockAllocator(64, 16)
    p = a.new_request()
    a.prefill(p, 32)
    kids = [a.fork(p) for _ in range(5)]
    a.release(p)
    for b in a.table(kids[0]):
        assert a.ref[b] == 5
    a.check_invariants()


def test_brute_force_against_private_copies():
    """Every sequence of <= 7 ops (new/append/fork/release, <= 3 live requests)
    on a 4-block pool with P = 2, explored depth first.

    After every op: the allocator invariants hold, and each live request's rows,
    read through its block table from the physical content the trace built,
    equal a naive model in which every request owns a private list of rows
    ("paged output equals private copies").  Row values are unique per write.
    """
    num_blocks, P, depth, max_live = 4, 2, 7, 3
    visited = [0]

    def check(a, live, private, content):
        a.check_invariants()
        for r in live:
            tab, T = a.table(r), a.length(r)
            got = [content.get(tab[t // P] * P + t % P) for t in range(T)]
            assert got == private[r]

    def step(a, live, private, content, next_val, op, r):
        if op == "new":
            rid = a.new_request()
            live.append(rid)
            private[rid] = []
        elif op == "append":
            n0 = len(a.trace)
            try:
                slot = a.append(r)
            except OutOfBlocks:
                return next_val
            for t in a.trace[n0:]:
                if t[0] == "copy":
                    for o in range(P):
                        src, dst = t[1] * P + o, t[2] * P + o
                        if src in content:
                            content[dst] = content[src]
                        else:
                            content.pop(dst, None)
            content[slot] = next_val
            private[r].append(next_val)
            return next_val + 1
        elif op == "fork":
            c = a.fork(r)
            live.append(c)
            private[c] = list(private[r])
        else:
            a.release(r)
            live.remove(r)
            del private[r]
        return next_val

    def dfs(a, live, private, content, next_val, d):
        visited[0] += 1
        check(a, live, private, content)
        if d == depth:
            return
        moves = [("new", None)] if len(live) < max_live else []
        for r in live:
            moves += [("append", r), ("release", r)]
            if len(live) < max_live:
                moves.append(("fork", r))
        for op, r in moves:
            a2 = copy.deepcopy(a)
            live2, private2, content2 = list(live), {k: list(v) for k, v in private.items()}, dict(content)
            nv = step(a2, live2, private2, content2, next_val, op, r)
            dfs(a2, live2, private2, content2, nv, d + 1)

    dfs(BlockAllocator(num_blocks, P), [], {}, {}, 1, 0)
    assert visited[0] > 20000


def test_trace_replay_on_bit_pool_matches_private_rows():
    """The same check through oracle.pool: replaying the trace on bit arrays."""
    rng = np.random.default_rng(7)
    a = BlockAllocator(12, 4, free_order=rng.permutation(12))
    r0 = a.new_request()
    a.prefill(r0, 6)
    r1 = a.fork(r0)
    a.prefill(r1, 3)
    a.prefill(r0, 2)
    r2 = a.fork(r1)
    a.append(r2)
    n_w = sum(1 for op in a.trace if op[0] == "write")
    k_rows = rng.integers(0, 1 << 16, size=(n_w, 2, 3), dtype=np.uint16)
    v_rows = rng.integers(0, 1 << 16, size=(n_w, 2, 3), dtype=np.uint16)
    pool = BitPool(np.zeros((12, 2, 4, 3), np.uint16), np.zeros((12, 2, 3, 4), np.uint16), "bf16")
    replay(pool, a.trace, k_rows, v_rows)
    # Private model: rows of each request in write order, inherited at fork.
    w_of = {}
    w = 0
    for op in a.trace:
        if op[0] == "write":
            w_of[(op[1], op[2])] = w
            w += 1
    hist = {r0: [w_of[(r0, t)] for t in range(6)] + [w_of[(r0, 6)], w_of[(r0, 7)]],
            r1: [w_of[(r0, t)] for t in range(6)] + [w_of[(r1, t)] for t in range(6, 9)]}
    hist[r2] = hist[r1] + [w_of[(r2, 9)]]
    for r, rows in hist.items():
        tab, T = a.table(r), a.length(r)
        for h in range(2):
            ks = np.stack([pool.k[tab[t // 4], h, t % 4, :] for t in range(T)])
            vs = np.stack([pool.v[tab[t // 4], h, :, t % 4] for t in range(T)])
            assert np.array_equal(ks, k_rows[rows, h])
            assert np.array_equal(vs, v_rows[rows, h])
