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


def suggest_partition_tokens(seq_lens: Sequence[int], num_kv_heads: int, num_cus: int = 256) -> int:
    """A partition length for ``paged_decode`` chosen from the lengths the
    caller knows (the library sees only the table width and the batch).

    Returns 0 (the library's own plan) unless the batch already gives every
    CU a (request, kv head) of its own and its longest request is far above
    the mean; then the long requests are cut near twice the mean length, so
    that they stop setting the kernel's duration while the short ones keep a
    single partition.  Measured on MI355X: a lognormal batch of 128 requests
    (median 100, max 8192 tokens) decodes in 62 us with 1024-token partitions
    against 102 us unsplit; uniform or mildly ragged batches are fastest
    unsplit.
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.size == 0 or lens.size * num_kv_heads < num_cus:
        return 0
    mean = float(lens.mean())
    longest = int(lens.max())
    if longest <= 4 * mean:
        return 0
    pt = int(-(-int(2 * mean) // 256) * 256)
    pt = max(512, pt)
    return 0 if pt >= longest else pt
