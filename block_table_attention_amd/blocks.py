"""Host-side block bookkeeping for callers of the library.

The library moves and reads bytes; choosing the physical block and slot of a
token is the caller's job.  ``BlockManager`` does that job for one cache group:

* Free blocks wait in a FIFO: allocation takes the head, and a block whose last
  reference goes away joins the tail ("Cache Concepts: Prefix Matching vs.
  Storage", the queue of empty blocks).
* A block's reference count is the number of request tables that map it
  ("M5.3 - KV Memory Layout and Exact Reuse", 0x04B).
* ``fork`` maps the same blocks into a new request; each gains a reference
  (0x05, 0x05B).
* An append at in-block offset o = T mod P (0x04E):
  * o == 0: takes a fresh block;
  * o > 0 with a private tail: writes in place;
  * o > 0 with a shared tail: first copies the tail into a fresh block, maps the
    copy in its place and drops one reference from the shared block
    (copy-on-write before divergence, 0x05B; "7. Memory Management and Local
    Model State", "Sharing and copy-on-write").
* ``release`` drops the request's references (0x05E).

Appends return the slot ids for ``kv_append`` and the (src, dst) pairs for
``block_copy``; the copies must be issued before the writes.  An append that
cannot get the blocks it needs raises ``OutOfBlocks`` and changes nothing.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = np.arange(num_blocks) if free_order is None else np.asarray(free_order)
        if order.shape != (num_blocks,) or not np.array_equal(np.sort(order), np.arange(num_blocks)):
            raise ValueError("free_order must be a permutation of all block ids")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self._free = deque(int(b) for b in order)
        self._ref = np.zeros(num_blocks, dtype=np.int64)
        self._tables: Dict[int, List[int]] = {}
        self._lens: Dict[int, int] = {}
        self._next_rid = 0

    # -- requests -----------------------------------------------------------
    def new_request(self) -> int:
        rid = self._next_rid
        self._next_rid += 1
        self._tables[rid] = []
        self._lens[rid] = 0
        return rid

    def fork(self, rid: int) -> int:
        child = self.new_request()
        table = list(self._tables[rid])
        self._tables[child] = table
        self._lens[child] = self._lens[rid]
        for b in table:
            self._ref[b] += 1
        return child

    def release(self, rid: int) -> None:
        table = self._tables.pop(rid)
        del self._lens[rid]
        for b in table:
            self._drop(b)

    def append(self, rid: int, n: int = 1) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Reserve positions T .. T+n-1 of request ``rid``.

        Returns (slots int64 [n], copies [(src, dst)]): issue ``block_copy`` of
        the copies, then ``kv_append`` of the rows at those slots.
        """
        if n < 0:
            raise ValueError("n must be non-negative")
        P = self.block_size
        table = self._tables[rid]
        T = self._lens[rid]
        if n == 0:
            return np.zeros(0, dtype=np.int64), []
        cow = T % P != 0 and self._ref[table[-1]] > 1
        fresh = -(-(T + n) // P) - len(table)
        if int(cow) + fresh > len(self._free):
            raise OutOfBlocks(f"request {rid} needs {int(cow) + fresh} blocks, "
                              f"{len(self._free)} free")
        copies: List[Tuple[int, int]] = []
        if cow:
            src = table[-1]
            dst = self._take()
            copies.append((src, dst))
            table[-1] = dst
            self._drop(src)
        for _ in range(fresh):
            table.append(self._take())
        pos = np.arange(T, T + n, dtype=np.int64)
        slots = np.asarray(table, dtype=np.int64)[pos // P] * P + pos % P
        self._lens[rid] = T + n
        return slots, copies

    def blocks_needed(self, rid: int, n: int) -> int:
        """Free blocks ``append(rid, n)`` would take (fresh blocks plus a
        copy-on-write destination)."""
        if n <= 0:
            return 0
        P = self.block_size
        table = self._tables[rid]
        T = self._lens[rid]
        cow = T % P != 0 and self._ref[table[-1]] > 1
        return int(cow) + -(-(T + n) // P) - len(table)

    # -- views ----------------------------------------------------------------
    def table(self, rid: int) -> List[int]:
        return list(self._tables[rid])

    def length(self, rid: int) -> int:
        return self._lens[rid]

    def ref(self, block: int) -> int:
        return int(self._ref[block])

    def n_free(self) -> int:
        return len(self._free)

    def block_tables(self, rids: Sequence[int], width: Optional[int] = None) -> np.ndarray:
        """int32 [len(rids), width] block tables, padded with -1."""
        need = max((len(self._tables[r]) for r in rids), default=0)
        width = max(need, 1) if width is None else width
        if width < need:
            raise ValueError(f"width {width} < {need} blocks")
        out = np.full((len(rids), width), -1, dtype=np.int32)
        for i, r in enumerate(rids):
            t = self._tables[r]
            out[i, :len(t)] = t
        return out

    def seq_lens(self, rids: Sequence[int]) -> np.ndarray:
        return np.array([self._lens[r] for r in rids], dtype=np.int32)

    # -- blocks -----------------------------------------------------------------
    def _take(self) -> int:
        b = self._free.popleft()
        self._ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self._ref[b] -= 1
        if self._ref[b] == 0:
            self._free.append(b)


class BundleManager:
    """Block bookkeeping for several cache groups ("M5.3", 0x03B: one pool
    and one block table per group; 0x04E-0x04F: an append reserves the blocks
    of every group before any group changes, so it succeeds in all groups or
    in none).  Group g has its own block size, pool size and free FIFO; a
    request has one length and one table per group.

    ``append`` returns, per group, the slots for ``kv_append_bundle`` and the
    (src, dst) pairs for ``block_copy_bundle``; issue the copies first.
    """

    def __init__(self, num_blocks: Sequence[int], block_sizes: Sequence[int],
                 free_orders: Optional[Sequence[Sequence[int]]] = None):
        if len(num_blocks) != len(block_sizes) or not num_blocks:
            raise ValueError("one pool size and block size per group")
        self.groups = [BlockManager(n, p, None if free_orders is None else free_orders[g])
                       for g, (n, p) in enumerate(zip(num_blocks, block_sizes))]

    def new_request(self) -> int:
        ids = {m.new_request() for m in self.groups}
        assert len(ids) == 1
        return ids.pop()

    def fork(self, rid: int) -> int:
        ids = {m.fork(rid) for m in self.groups}
        assert len(ids) == 1
        return ids.pop()

    def release(self, rid: int) -> None:
        for m in self.groups:
            m.release(rid)

    def append(self, rid: int, n: int = 1):
        """Reserve positions T .. T+n-1 in every group: ([slots per group],
        [copies per group]); raises OutOfBlocks with no group changed."""
        for g, m in enumerate(self.groups):
            need = m.blocks_needed(rid, n)
            if need > m.n_free():
                raise OutOfBlocks(f"group {g}: request {rid} needs {need} blocks, "
                                  f"{m.n_free()} free")
        out = [m.append(rid, n) for m in self.groups]
        return [o[0] for o in out], [o[1] for o in out]

    def length(self, rid: int) -> int:
        return self.groups[0].length(rid)

    def block_tables(self, rids: Sequence[int]) -> List[np.ndarray]:
        return [m.block_tables(rids) for m in self.groups]

    def seq_lens(self, rids: Sequence[int]) -> np.ndarray:
        return self.groups[0].seq_lens(rids)


PARTITIONS_BALANCED = -1   # the library's balanced decomposition (PBA_PARTITIONS_BALANCED)


def suggest_partition_tokens(seq_lens: Sequence[int], num_kv_heads: int, num_cus: int = 256,
                             balanced_ok: bool = True) -> int:
    """A partition choice for ``paged_decode`` from the lengths the caller
    knows (the library sees only the table width and the batch).

    * Very ragged batches -- every CU already has a (request, kv head) and the
      longest request is over 4x the mean -- get the balanced decomposition
      (``PARTITIONS_BALANCED``: the batch's chunks spread evenly over the CUs)
      when ``balanced_ok`` (bf16 pools, at most 2048 rows), else partitions of
      about twice the mean length.  Lognormal batches of 128 requests (median
      100, max 8192 tokens): 50 / 49 / 50 us at P = 16 / 64 / 256 balanced,
      61 / 77 / 76 us with 1024-token partitions, 102 / 139 / 140 us unsplit.
    * Mildly ragged batches (longest over 1.3x the mean and at least 1536
      tokens) with more (request, kv head) pairs than half the CUs get 512-token
      partitions (1024 from 4096 tokens on): one work-group streams at most
      ~60 GB/s from its CU, and with whole rows per work-group the CUs that
      hold the longest rows finish last.  Measured 4-16 % faster over a grid
      of batches (8-128 requests, 4-8 kv heads, rows up to 8192 tokens), e.g.
      a 32-layer bundle of 40 requests of 101-2028 tokens at 4 kv heads:
      26.7 -> 21.3 us per layer.
    * Otherwise 0, the library's plan (uniform batches are fastest with it,
      and so are batches that fill under half the CUs, which it splits).
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.size == 0:
        return 0
    units = lens.size * num_kv_heads
    mean = float(lens.mean())
    longest = int(lens.max())
    if units >= num_cus and longest > 4 * mean:
        if balanced_ok and lens.size <= 2048:
            return PARTITIONS_BALANCED
        pt = int(-(-int(2 * mean) // 256) * 256)
        pt = max(512, pt)
        return 0 if pt >= longest else pt
    if 2 * units > num_cus and longest > 1.3 * mean and longest >= 1536:
        return 512 if longest < 4096 else 1024
    return 0


# ---------------------------------------------------------------------------
# Shared-prefix execution plans ("M5.3", 0x0BB-0x0BE)
# ---------------------------------------------------------------------------
def sharing_order(tables: np.ndarray) -> np.ndarray:
    """A batch order in which rows that map the same leading blocks are
    adjacent (lexicographic order of the block tables), so that each shared
    chunk covers one contiguous range of rows."""
    t = np.asarray(tables)
    return np.lexsort(t.T[::-1]).astype(np.int64)


def shared_chunks(tables: np.ndarray, seq_lens: Sequence[int], block_size: int,
                  threshold: int = 1):
    """Chunks of a batch, in tree pre-order, and each row's first private token.

    A chunk (row_begin, row_end, tok_begin, tok_end) is a maximal run of whole,
    fully visible blocks that every row of [row_begin, row_end) maps to the same
    physical ids, below the chunks of its ancestors; only runs covering more
    than ``threshold`` rows become chunks (0x0BD's coverage threshold).  Rows
    sharing leading blocks must be adjacent (see ``sharing_order``).
    """
    t = np.asarray(tables)
    lens = np.asarray(seq_lens, dtype=np.int64)
    P = block_size
    full = lens // P                         # whole blocks each row can see
    B = len(lens)
    chunks = []
    private = np.zeros(B, dtype=np.int64)

    def visit(a: int, b: int, j0: int) -> None:
        if b - a <= threshold:
            private[a:b] = j0 * P
            return
        lim = int(full[a:b].min())
        j = j0
        while j < lim and bool((t[a:b, j] == t[a, j]).all()):
            j += 1
        if j > j0:
            chunks.append((a, b, j0 * P, j * P))
        r = a
        while r < b:
            if full[r] <= j:
                private[r] = j * P
                r += 1
                continue
            e = r + 1
            while e < b and full[e] > j and t[e, j] == t[r, j]:
                e += 1
            visit(r, e, j)
            r = e

    visit(0, B, 0)
    return chunks, private


@dataclass
class HostSharedPlan:
    items: np.ndarray          # int32 [n, 8]: row0, nrows, tb, te, slot, tiles, 0, 0
    row_private: np.ndarray    # int32 [B, 2]: first private token, its slot
    max_slots: int
    partition_tokens: int
    chunks: List[Tuple[int, int, int, int]]
    private_parts: int = 0     # most private pieces of any row
    private_tokens: int = 0    # most private positions of any row (0: none given)


def shared_plan(tables: np.ndarray, seq_lens: Sequence[int], block_size: int, group: int,
                partition_tokens: int = 256, threshold: int = 1,
                tiles_per_item: int = 4) -> HostSharedPlan:
    """The work items of ``paged_decode_shared`` for a batch.

    Every chunk is cut into pieces of ``partition_tokens`` keys from its first
    key; each piece is one partial state (slot) of every row it covers.  Rows
    of a piece go in 16-column tiles of 16 // group rows, up to
    ``tiles_per_item`` (1, 2 or 4) tiles per item: one K/V read serves them
    all (tiles go in groups of two whose waves split the keys).  A row's
    slots: its chunks' pieces in path order, then its private pieces.  The
    plan also bounds every row's private positions, which lets the library
    walk short private ranges four rows per work-group.
    """
    if tiles_per_item not in (1, 2, 4):
        raise ValueError("tiles_per_item must be 1, 2 or 4")
    if partition_tokens <= 0 or partition_tokens % 256:
        raise ValueError("partition_tokens must be a positive multiple of 256")
    lens = np.asarray(seq_lens, dtype=np.int64)
    chunks, private = shared_chunks(tables, lens, block_size, threshold)
    pt = partition_tokens
    rpt = 16 // group
    if rpt < 1:
        raise ValueError("group (q-heads per kv head) must be at most 16")
    next_slot = np.zeros(len(lens), dtype=np.int64)
    items = []
    for a, b, t0, t1 in chunks:
        base = int(next_slot[a])
        if not (next_slot[a:b] == base).all():
            raise AssertionError("rows of a chunk disagree on their ancestors")
        pieces = -(-(t1 - t0) // pt)
        tiles = -(-(b - a) // rpt)
        for k in range(pieces):
            tb = t0 + k * pt
            te = min(t1, tb + pt)
            ti = 0
            while ti < tiles:
                left = tiles - ti
                n_t = min(tiles_per_item, 4 if left >= 4 else (2 if left >= 2 else 1))
                row0 = a + ti * rpt
                nrows = min(b, a + (ti + n_t) * rpt) - row0
                items.append((row0, nrows, tb, te, base + k, n_t, 0, 0))
                ti += n_t
        next_slot[a:b] += pieces
    row_private = np.stack([private, next_slot], axis=1).astype(np.int32)
    priv_pieces = -(-np.maximum(lens - private, 0) // pt)
    max_slots = int(max(1, (next_slot + priv_pieces).max()))
    arr = np.array(items, dtype=np.int32).reshape(-1, 8)
    # The launch holds one grid plane per possible private piece; the true
    # bound keeps it from filling with empty work-groups.
    return HostSharedPlan(arr, row_private, max_slots, pt, chunks,
                          int(max(1, priv_pieces.max())),
                          int(max(1, np.maximum(lens - private, 0).max())))
