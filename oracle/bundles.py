"""Cache groups with a layer axis, and whole-bundle appends and copies.

Test infrastructure only (see ``oracle/__init__.py``).

Follows "M5.3 - KV Memory Layout and Exact Reuse":
  * 0x03B: every cache group has its own pool and its own block table per
    request; a group's token row spans all of its layers, so its row bytes are
    B_row,g = L_g H_g d_g (b_K + b_V), and one all-layer block of the request
    is an accounting bundle of one block per group, P_g B_row,g bytes in each.
    Group block sizes may differ, so block and offset are computed per group.
  * 0x03C-0x03E: layer l of group g is the group-local index l - L_g,start;
    the element offset of (layer, block, head, token, dim) is the dot product
    of the coordinate, taken in the group's declared axis order, with the
    row-major strides of that order.  A group may be layer major (one block's
    layers far apart) or block major (one block's layers adjacent).
  * 0x04E: an append at offset o = T mod P_g takes a fresh block in every group
    that crosses a boundary, writes in place in a group whose tail is private,
    and copies a shared tail first; the new row is written in every group.
  * 0x04F: the destinations of every group are reserved before anything is
    published; a failure after some groups were reserved returns those
    reservations and leaves the committed state exactly as it was.
  * 0x05B-0x05C: a divergent append into a shared tail bundle copies the tail
    block of every group whose tail is shared and publishes all groups'
    replacements at once; a successor that moves only some groups (a half
    bundle) is invalid.

The pools hold raw scalar bits in flat arrays addressed through the manifest's
stride rule, so they compare byte for byte with any device buffer described
by the same axis order.
"""
from __future__ import annotations

import hashlib
from collections import deque
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .allocator import OutOfBlocks
from .bits import BITS_DTYPE, SCALAR_BYTES
from .layout import row_major_strides
from .pool import BitPool

AXES = ("layer", "block", "head", "token", "dim")
LAYER_MAJOR_K = ("layer", "block", "head", "token", "dim")
LAYER_MAJOR_V = ("layer", "block", "head", "dim", "token")
BLOCK_MAJOR_K = ("block", "layer", "head", "token", "dim")
BLOCK_MAJOR_V = ("block", "layer", "head", "dim", "token")


class HalfBundle(ValueError):
    """A write or copy that would move some cache groups but not the others."""


class InjectedFailure(RuntimeError):
    """Raised by ``BundleAllocator.append(fail_at_group=g)`` before group g reserves."""


@dataclass(frozen=True)
class GroupManifest:
    """Layout of one cache group: sizes and the K and V axis orders (0x03E)."""

    layers: int
    num_blocks: int
    block_size: int
    kv_heads: int
    head_dim: int
    dtype: str
    k_axes: Tuple[str, ...] = LAYER_MAJOR_K
    v_axes: Tuple[str, ...] = LAYER_MAJOR_V

    def __post_init__(self):
        for axes in (self.k_axes, self.v_axes):
            if sorted(axes) != sorted(AXES):
                raise ValueError(f"axis order {axes} is not a permutation of {AXES}")

    def extent(self, axis: str) -> int:
        return {"layer": self.layers, "block": self.num_blocks, "head": self.kv_heads,
                "token": self.block_size, "dim": self.head_dim}[axis]

    def shape(self, kind: str) -> Tuple[int, ...]:
        axes = self.k_axes if kind == "K" else self.v_axes
        return tuple(self.extent(a) for a in axes)

    def strides(self, kind: str) -> Dict[str, int]:
        """Element stride of every named axis in the K or V tensor."""
        axes = self.k_axes if kind == "K" else self.v_axes
        return dict(zip(axes, row_major_strides(self.shape(kind))))

    def elements(self) -> int:
        n = 1
        for a in AXES:
            n *= self.extent(a)
        return n


class LayeredPool:
    """One cache group's K and V as flat arrays of scalar bits."""

    def __init__(self, manifest: GroupManifest, k_bits: np.ndarray, v_bits: np.ndarray):
        m = manifest
        n = m.elements()
        k = np.asarray(k_bits).reshape(-1)
        v = np.asarray(v_bits).reshape(-1)
        if k.size != n or v.size != n:
            raise ValueError(f"pool arrays must hold {n} scalars")
        self.m = m
        self.k = np.array(k, dtype=BITS_DTYPE[m.dtype], copy=True)
        self.v = np.array(v, dtype=BITS_DTYPE[m.dtype], copy=True)

    # -- addressing (0x03C-0x03E) -------------------------------------------
    def offsets(self, kind: str, layer, block, head, token, dim) -> np.ndarray:
        """Element offsets of broadcast coordinate arrays in the K or V tensor."""
        s = self.m.strides(kind)
        return (np.asarray(layer, np.int64) * s["layer"] + np.asarray(block, np.int64) * s["block"]
                + np.asarray(head, np.int64) * s["head"] + np.asarray(token, np.int64) * s["token"]
                + np.asarray(dim, np.int64) * s["dim"])

    def _grid(self):
        m = self.m
        L = np.arange(m.layers)[:, None, None]
        H = np.arange(m.kv_heads)[None, :, None]
        C = np.arange(m.head_dim)[None, None, :]
        return L, H, C

    # -- physical operations ----------------------------------------------------
    def kv_append(self, slots: Sequence[int], k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        """Row i (bits [layers, heads, dim]) of every layer goes to slot s_i:
        block s_i div P, offset s_i mod P; a negative slot skips (0x03D)."""
        m = self.m
        slots = np.asarray(slots, dtype=np.int64)
        k_rows = np.asarray(k_rows)
        v_rows = np.asarray(v_rows)
        shape = (len(slots), m.layers, m.kv_heads, m.head_dim)
        if k_rows.shape != shape or v_rows.shape != shape:
            raise ValueError(f"rows must be {shape}")
        live = slots[slots >= 0]
        if len(np.unique(live)) != len(live):
            raise ValueError("duplicate slot in one append")
        if live.size and live.max() >= m.num_blocks * m.block_size:
            raise ValueError("slot outside the pool")
        L, H, C = self._grid()
        for i, s in enumerate(slots.tolist()):
            if s < 0:
                continue
            blk, off = divmod(s, m.block_size)
            self.k[self.offsets("K", L, blk, H, off, C)] = k_rows[i]
            self.v[self.offsets("V", L, blk, H, off, C)] = v_rows[i]

    def block_copy(self, src: Sequence[int], dst: Sequence[int]) -> None:
        """Whole blocks: every layer, head, row and dim of K and V (0x05B)."""
        m = self.m
        src = [int(b) for b in src]
        dst = [int(b) for b in dst]
        self.check_pairs(src, dst)
        L = np.arange(m.layers)[:, None, None, None]
        H = np.arange(m.kv_heads)[None, :, None, None]
        T = np.arange(m.block_size)[None, None, :, None]
        C = np.arange(m.head_dim)[None, None, None, :]
        for s, d in zip(src, dst):
            for kind, arr in (("K", self.k), ("V", self.v)):
                arr[self.offsets(kind, L, d, H, T, C)] = arr[self.offsets(kind, L, s, H, T, C)]

    def check_pairs(self, src: Sequence[int], dst: Sequence[int]) -> None:
        src = [int(b) for b in src]
        dst = [int(b) for b in dst]
        if len(src) != len(dst):
            raise ValueError("one destination per source")
        if len(set(dst)) != len(dst) or set(src) & set(dst):
            raise ValueError("overlapping copy pairs")
        if any(not 0 <= b < self.m.num_blocks for b in src + dst):
            raise ValueError("block id outside the pool")

    # -- reads ------------------------------------------------------------------
    def layer_pool(self, layer: int) -> BitPool:
        """Layer ``layer`` as a single-layer pool (K [NB, H, P, d], V [NB, H, d, P])."""
        m = self.m
        B = np.arange(m.num_blocks)[:, None, None, None]
        H = np.arange(m.kv_heads)[None, :, None, None]
        T = np.arange(m.block_size)[None, None, :, None]
        C = np.arange(m.head_dim)[None, None, None, :]
        k = self.k[self.offsets("K", layer, B, H, T, C)]
        v = self.v[self.offsets("V", layer, B, H, T, C)].transpose(0, 1, 3, 2)
        return BitPool(k, v, m.dtype)

    def digest(self) -> str:
        h = hashlib.sha256()
        h.update(self.k.tobytes())
        h.update(self.v.tobytes())
        return h.hexdigest()


def row_bytes(m: GroupManifest) -> int:
    """B_row,g from the pool's own size: bytes of K and V per token slot."""
    return (m.elements() * 2 * SCALAR_BYTES[m.dtype]) // (m.num_blocks * m.block_size)


def bundle_bytes(groups: Sequence[GroupManifest]) -> int:
    """B_bundle = sum_g P_g B_row,g (0x04E)."""
    return sum(m.block_size * row_bytes(m) for m in groups)


def bundle_append(pools: Sequence[LayeredPool], slots: Sequence[Sequence[int]],
                  k_rows: Sequence[np.ndarray], v_rows: Sequence[np.ndarray]) -> None:
    """Append token i to every group at its group's slot; a token whose slot is
    negative in some groups and not in others is a half bundle (0x04E, 0x05C),
    rejected before any group changes."""
    n = {len(s) for s in slots}
    if len(n) != 1 or len(slots) != len(pools):
        raise HalfBundle("every group needs one slot per token")
    S = np.asarray([np.asarray(s, dtype=np.int64) for s in slots])
    skip = S < 0
    if (skip.any(axis=0) & ~skip.all(axis=0)).any():
        raise HalfBundle("a token is written to some groups only")
    for p, s, k, v in zip(pools, slots, k_rows, v_rows):
        p.kv_append(s, k, v)


def bundle_copy(pools: Sequence[LayeredPool], pairs: Sequence[Sequence[Tuple[int, int]]]) -> None:
    """The copies of one publication, every group's pairs at once: all pairs
    of all groups are checked before any group changes, so a bad pair in one
    group leaves every group as it was (no half-published successor, 0x05C).
    Groups may copy different numbers of blocks when their block sizes differ
    (a tail can be shared in one group while another starts a fresh block)."""
    if len(pairs) != len(pools):
        raise HalfBundle("one pair list per group")
    for p, pr in zip(pools, pairs):
        p.check_pairs([s for s, _ in pr], [d for _, d in pr])
    for p, pr in zip(pools, pairs):
        if len(pr):
            p.block_copy([s for s, _ in pr], [d for _, d in pr])


class BundleAllocator:
    """Free-FIFO allocator over several cache groups: one FIFO, reference
    counts and block table per group, one length per request.

    ``append`` reserves every group's destination in group order, then
    publishes all of them; a failure during reservation returns the reserved
    blocks to the heads of their FIFOs in reverse order, so the committed
    state is unchanged (0x04F).  The trace records, per appended token, the
    copies ``("copy", group, src, dst)`` of every group, then the writes
    ``("write", group, request, position, slot)`` of every group.
    """

    def __init__(self, num_blocks: Sequence[int], block_sizes: Sequence[int],
                 free_orders: Optional[Sequence[Sequence[int]]] = None):
        if len(num_blocks) != len(block_sizes) or not num_blocks:
            raise ValueError("one block count and block size per group")
        self.G = len(num_blocks)
        self.P = [int(p) for p in block_sizes]
        self.free: List[deque] = []
        for g, n in enumerate(num_blocks):
            order = list(range(n)) if free_orders is None else [int(b) for b in free_orders[g]]
            if sorted(order) != list(range(n)):
                raise ValueError("free order must be a permutation of the group's block ids")
            self.free.append(deque(order))
        self.ref: List[List[int]] = [[0] * int(n) for n in num_blocks]
        self.tables: Dict[int, List[List[int]]] = {}
        self.lengths: Dict[int, int] = {}
        self.trace: List[Tuple] = []
        self._next = 0

    def new_request(self) -> int:
        rid = self._next
        self._next += 1
        self.tables[rid] = [[] for _ in range(self.G)]
        self.lengths[rid] = 0
        return rid

    def fork(self, rid: int) -> int:
        child = self.new_request()
        self.tables[child] = [list(t) for t in self.tables[rid]]
        self.lengths[child] = self.lengths[rid]
        for g, t in enumerate(self.tables[child]):
            for b in t:
                self.ref[g][b] += 1
        return child

    def release(self, rid: int) -> None:
        for g, t in enumerate(self.tables.pop(rid)):
            for b in t:
                self._drop(g, b)
        del self.lengths[rid]

    def _drop(self, g: int, b: int) -> None:
        self.ref[g][b] -= 1
        if self.ref[g][b] == 0:
            self.free[g].append(b)

    def append(self, rid: int, fail_at_group: Optional[int] = None) -> List[int]:
        """Append one token at position T; returns the slot of each group."""
        T = self.lengths[rid]
        tables = self.tables[rid]
        # What each group needs (0x04E): a fresh block, a copy, or nothing.
        needs = []
        for g in range(self.G):
            j, o = divmod(T, self.P[g])
            if o == 0:
                if len(tables[g]) != j:
                    raise RuntimeError("table length drifted from ceil(T/P)")
                needs.append("fresh")
            elif self.ref[g][tables[g][-1]] > 1:
                needs.append("copy")
            else:
                needs.append(None)
        # Reserve in group order; undo on failure (0x04F).
        reserved: List[Tuple[int, int]] = []
        try:
            for g in range(self.G):
                if fail_at_group == g:
                    raise InjectedFailure(f"failure before group {g} reserves")
                if needs[g] is None:
                    continue
                if not self.free[g]:
                    raise OutOfBlocks(f"group {g} has no free block")
                reserved.append((g, self.free[g].popleft()))
        except (InjectedFailure, OutOfBlocks):
            for g, b in reversed(reserved):
                self.free[g].appendleft(b)
            raise
        # Publish every group (0x05C).
        got = dict(reserved)
        writes = []
        for g in range(self.G):
            t = tables[g]
            j, o = divmod(T, self.P[g])
            if needs[g] == "fresh":
                t.append(got[g])
                self.ref[g][got[g]] = 1
            elif needs[g] == "copy":
                src = t[-1]
                self.trace.append(("copy", g, src, got[g]))
                t[-1] = got[g]
                self.ref[g][got[g]] = 1
                self._drop(g, src)
            writes.append(t[j] * self.P[g] + o)
        for g in range(self.G):
            self.trace.append(("write", g, rid, T, writes[g]))
        self.lengths[rid] = T + 1
        return writes

    def prefill(self, rid: int, n: int) -> List[List[int]]:
        return [self.append(rid) for _ in range(n)]

    def table(self, rid: int, g: int) -> List[int]:
        return list(self.tables[rid][g])

    def state_digest(self) -> str:
        h = hashlib.sha256()
        h.update(repr([list(f) for f in self.free]).encode())
        h.update(repr(self.ref).encode())
        h.update(repr(sorted((r, t) for r, t in self.tables.items())).encode())
        h.update(repr(sorted(self.lengths.items())).encode())
        return h.hexdigest()

    def check_invariants(self) -> None:
        for g in range(self.G):
            counted = [0] * len(self.ref[g])
            for ts in self.tables.values():
                for b in ts[g]:
                    counted[b] += 1
            if counted != self.ref[g]:
                raise RuntimeError(f"group {g}: refcounts differ from reachability")
            free = set(self.free[g])
            if len(free) != len(self.free[g]):
                raise RuntimeError(f"group {g}: duplicate free block")
            for b, r in enumerate(self.ref[g]):
                if (b in free) != (r == 0):
                    raise RuntimeError(f"group {g}: block {b} free/live mismatch")


def replay_bundle_trace(pools: Sequence[LayeredPool], trace: Sequence[Tuple],
                        k_rows: Sequence[np.ndarray], v_rows: Sequence[np.ndarray]) -> None:
    """Apply a ``BundleAllocator`` trace token by token: the copies of every
    group, then the writes of every group; write number w of group g takes
    row w of ``k_rows[g]`` / ``v_rows[g]`` (bits [n, layers, heads, dim])."""
    G = len(pools)
    w = [0] * G
    i = 0
    while i < len(trace):
        copies: List[List[Tuple[int, int]]] = [[] for _ in range(G)]
        while i < len(trace) and trace[i][0] == "copy":
            _, g, s, d = trace[i]
            copies[g].append((s, d))
            i += 1
        if any(copies):
            for g in range(G):
                if copies[g]:
                    pools[g].block_copy([s for s, _ in copies[g]], [d for _, d in copies[g]])
        seen = set()
        while i < len(trace) and trace[i][0] == "write" and trace[i][1] not in seen:
            _, g, _, _, slot = trace[i]
            seen.add(g)
            pools[g].kv_append([slot], k_rows[g][w[g]:w[g] + 1], v_rows[g][w[g]:w[g] + 1])
            w[g] += 1
            i += 1
        if seen and len(seen) != G:
            raise HalfBundle("a token was written to some groups only")
        if i < len(trace) and trace[i][0] not in ("copy", "write"):
            raise ValueError(trace[i])
