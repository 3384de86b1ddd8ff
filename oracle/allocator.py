"""Free-FIFO block pool with reference counts, fork, append and copy-on-write.

Test infrastructure only (see ``oracle/__init__.py``).

Follows:
  * "M5.3 - KV Memory Layout and Exact Reuse", 0x04B (a reference count equals
    the number of committed request-map references to the block; every
    reachable block has a positive count), 0x04C (fork, append, free), 0x04E
    (the three physical append paths), 0x05 / 0x05B (fork makes every mapped
    block shared; a divergent append into a shared partial tail copies it first,
    then writes; the old tail loses one reference), 0x05E (release drops the
    request's references), 0x09C (a prefix that ends on a block boundary needs
    no copy: the next append takes a fresh block), and the "Append And
    Copy-On-Write Edge Case" of 0x0AC.
  * "Cache Concepts: Prefix Matching vs. Storage": empty blocks wait in a FIFO;
    allocation takes the head, a freed block joins the tail.
  * "7. Memory Management and Local Model State", "Sharing and copy-on-write".

The allocator is single threaded and applies each operation atomically: a
failed allocation raises ``OutOfBlocks`` before any state changes, so the
predecessor state is preserved (0x05G).  Copy-on-write copies the whole
physical block (every row, every head, K and V); the rows a request may read
are the same under a copy of only the valid rows.

Every physical effect is recorded in ``trace`` in program order:
  ``("copy", src_block, dst_block)``  then
  ``("write", request_id, token_position, slot_id)``.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(RuntimeError):
    pass


class AllocatorError(RuntimeError):
    pass


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of all block ids")
        self.num_blocks = num_blocks
        self.P = block_size
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        self.trace: List[Tuple] = []
        self._next_rid = 0

    # -- block ownership ---------------------------------------------------
    def _alloc(self) -> int:
        if not self.free:
            raise OutOfBlocks("free FIFO is empty")
        b = self.free.popleft()
        if self.ref[b] != 0:
            raise AllocatorError(f"block {b} in free FIFO with ref {self.ref[b]}")
        self.ref[b] = 1
        return b

    def _incref(self, b: int) -> None:
        if self.ref[b] <= 0:
            raise AllocatorError(f"incref of unowned block {b}")
        self.ref[b] += 1

    def _decref(self, b: int) -> None:
        if self.ref[b] <= 0:
            raise AllocatorError(f"refcount underflow on block {b}")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    # -- request operations --------------------------------------------------
    def new_request(self) -> int:
        rid = self._next_rid
        self._next_rid += 1
        self.tables[rid] = []
        self.lengths[rid] = 0
        return rid

    def append(self, rid: int) -> int:
        """Append one token to request ``rid``; return the slot it is written to.

        With T the current length: o = T mod P.
          o == 0                 -> take a fresh block from the FIFO head;
          o > 0, tail ref == 1   -> write in place;
          o > 0, tail ref > 1    -> copy the tail into a fresh block, map it in
                                    place of the shared one, drop one reference
                                    from the shared block, then write.
        """
        table = self.tables[rid]
        T = self.lengths[rid]
        j, o = divmod(T, self.P)
        if o == 0:
            if len(table) != j:
                raise AllocatorError("table length drifted from ceil(T/P)")
            table.append(self._alloc())
        else:
            tail = table[-1]
            if self.ref[tail] > 1:
                dst = self._alloc()  # raises before any mutation
                self.trace.append(("copy", tail, dst))
                table[-1] = dst
                self._decref(tail)
        slot = table[j] * self.P + o
        self.trace.append(("write", rid, T, slot))
        self.lengths[rid] = T + 1
        return slot

    def prefill(self, rid: int, n: int) -> List[int]:
        return [self.append(rid) for _ in range(n)]

    def fork(self, rid: int) -> int:
        """The child maps the same blocks; every mapped block gains a reference."""
        child = self.new_request()
        self.tables[child] = list(self.tables[rid])
        self.lengths[child] = self.lengths[rid]
        for b in self.tables[child]:
            self._incref(b)
        return child

    def release(self, rid: int) -> None:
        for b in self.tables.pop(rid):
            self._decref(b)
        del self.lengths[rid]

    # -- views ---------------------------------------------------------------
    def table(self, rid: int) -> List[int]:
        return list(self.tables[rid])

    def length(self, rid: int) -> int:
        return self.lengths[rid]

    def n_free(self) -> int:
        return len(self.free)

    def n_live(self) -> int:
        return sum(1 for r in self.ref if r > 0)

    def state_key(self) -> Tuple:
        """Hashable snapshot of the whole committed state."""
        return (tuple(self.free), tuple(self.ref),
                tuple(sorted((r, tuple(t)) for r, t in self.tables.items())),
                tuple(sorted(self.lengths.items())), len(self.trace))

    def check_invariants(self) -> None:
        """Reachability refcounts, pool conservation, table length (0x04B, 0x0CF)."""
        counted = [0] * self.num_blocks
        for t in self.tables.values():
            for b in t:
                counted[b] += 1
        if counted != self.ref:
            raise AllocatorError("refcount differs from request-map reachability")
        if len(set(self.free)) != len(self.free):
            raise AllocatorError("duplicate block in free FIFO")
        free_set = set(self.free)
        for b in range(self.num_blocks):
            if (b in free_set) != (self.ref[b] == 0):
                raise AllocatorError(f"block {b} free/live mismatch")
        if self.n_free() + self.n_live() != self.num_blocks:
            raise AllocatorError("N_free + N_live != N_pool")
        for rid, t in self.tables.items():
            T = self.lengths[rid]
            if len(t) != -(-T // self.P):
                raise AllocatorError(f"request {rid}: table length != ceil(T/P)")
