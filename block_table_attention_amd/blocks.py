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


# ---------------------------------------------------------------------------
# Planning: thin wrappers over the library's host planners (libpba.so), which
# hold the decisions; these only convert between numpy arrays and the ABI.
# ---------------------------------------------------------------------------
def suggest_partition_tokens(seq_lens: Sequence[int], num_kv_heads: int,
                             balanced_ok: bool = True, num_q_heads: int = 0,
                             head_dim: int = 128) -> int:
    """The partition request the library chooses for a batch with these
    lengths (``pba_paged_decode_plan_ex`` with ``PBA_PARTITIONS_AUTO``): the
    balanced decomposition for very ragged batches that fill the CUs (or
    partitions of about twice the mean where it is not built: fp32 pools,
    ``balanced_ok`` False, more than 2048 rows), 512/1024-token partitions
    for mildly ragged ones, otherwise 0 (the library's table-width plan).
    The pool is described by its kv heads (q heads default to 4 per kv
    head), bf16 when ``balanced_ok`` else fp32."""
    import block_table_attention_amd as pba

    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.size == 0:
        return 0
    P = 16
    desc = pba.PoolDesc(k=0x10000, v=0x20000, dtype=1 if balanced_ok else 0, num_blocks=1,
                        block_size=P, num_kv_heads=num_kv_heads, head_dim=head_dim,
                        split_log2=0, k_stride_block=num_kv_heads * P * head_dim,
                        k_stride_head=P * head_dim, v_stride_block=num_kv_heads * P * head_dim,
                        v_stride_head=P * head_dim)
    width = max(1, int(-(-int(lens.max()) // P)))
    plan = pba.paged_decode_plan_ex(desc, num_q_heads or 4 * num_kv_heads, int(lens.size), width,
                                    pba.PARTITIONS_AUTO, lens)
    return plan["partition_request"]


# ---------------------------------------------------------------------------
# Shared-prefix execution plans ("M5.3", 0x0BB-0x0BE)
# ---------------------------------------------------------------------------
def sharing_order(tables: np.ndarray) -> np.ndarray:
    """A batch order in which rows that map the same leading blocks are
    adjacent (lexicographic order of the block tables, stable), so that each
    shared chunk covers one contiguous range of rows."""
    import block_table_attention_amd as pba

    t = np.asarray(tables)
    return pba.shared_plan_build(t, np.zeros(t.shape[0], np.int32), 16, 1)["order"]


def shared_chunks(tables: np.ndarray, seq_lens: Sequence[int], block_size: int,
                  threshold: int = 1):
    """Chunks of a batch, in tree pre-order, and each row's first private token.

    A chunk (row_begin, row_end, tok_begin, tok_end) is a maximal run of whole,
    fully visible blocks that every row of [row_begin, row_end) maps to the same
    physical ids, below the chunks of its ancestors; only runs covering more
    than ``threshold`` rows become chunks (0x0BD's coverage threshold).  Rows
    sharing leading blocks must be adjacent (see ``sharing_order``).
    """
    import block_table_attention_amd as pba

    r = pba.shared_plan_build(tables, seq_lens, block_size, 1, 256, threshold, 1)
    _require_identity(r["order"])
    return ([tuple(int(x) for x in c) for c in r["chunks"]],
            r["row_private"][:, 0].astype(np.int64))


def _require_identity(order: np.ndarray) -> None:
    if not np.array_equal(order, np.arange(order.size)):
        raise ValueError("rows sharing leading blocks must be adjacent: order the batch with "
                         "sharing_order first")


@dataclass
class HostSharedPlan:
    items: np.ndarray          # int32 [n, 8]: row0, nrows, tb, te, slot, tiles, 0, 0
    row_private: np.ndarray    # int32 [B, 2]: first private token, its slot
    max_slots: int
    partition_tokens: int
    chunks: List[Tuple[int, int, int, int]]
    private_parts: int = 0     # most private pieces of any row
    private_tokens: int = 0    # most private positions of any row (0: none given)
    kv_rows_read: int = 0      # key positions read per kv head (library ledger)
    chunk_visits: int = 0      # 32-token chunk reads per kv head
    partial_states: int = 0    # (row, slot) partial states written per kv head


def shared_plan(tables: np.ndarray, seq_lens: Sequence[int], block_size: int, group: int,
                partition_tokens: int = 256, threshold: int = 1,
                tiles_per_item: int = 4) -> HostSharedPlan:
    """The work items of ``paged_decode_shared`` for a batch already in
    sharing order (``pba_shared_plan_build``): every chunk cut into pieces of
    ``partition_tokens`` keys, its rows in 16-column tiles of 16 // group rows,
    up to ``tiles_per_item`` tiles per item; each row's private range after
    its last chunk; the plan's bounds and ledgers."""
    import block_table_attention_amd as pba

    if tiles_per_item not in (1, 2, 4):
        raise ValueError("tiles_per_item must be 1, 2 or 4")
    if partition_tokens <= 0 or partition_tokens % 256:
        raise ValueError("partition_tokens must be a positive multiple of 256")
    if not 1 <= group <= 16:
        raise ValueError("group (q-heads per kv head) must be at most 16")
    r = pba.shared_plan_build(tables, seq_lens, block_size, group, partition_tokens, threshold,
                              tiles_per_item)
    _require_identity(r["order"])
    return HostSharedPlan(r["items"].reshape(-1, 8), r["row_private"], r["max_slots"],
                          r["partition_tokens"], [tuple(int(x) for x in c) for c in r["chunks"]],
                          r["private_parts"], r["private_tokens"], r["kv_rows_read"],
                          r["chunk_visits"], r["partial_states"])
