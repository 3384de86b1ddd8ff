"""Contiguous virtual K/V (vAttention): address algebra, page ledgers, the
slot/page lifecycle, and decode over a request slot's contiguous rows.

Test infrastructure only (see ``oracle/__init__.py``).

Follows "M5.3 - KV Memory Layout and Exact Reuse":
  * 0x06A: one token row of one K or V tensor of one layer is
    B_row = H_kv d_h b bytes; a physical page group of G bytes holds G / B_row
    rows; a request slot's subrange of one tensor is R = G ceil(T_max B_row / G)
    bytes; the reservation is M_VA = 2 L B R; the handle pool is N_handle G; a
    request-page bundle (page q of every K and V tensor of every layer) is
    2 L G bytes; a slot needs ceil(T / P_tokens) mapped pages.  Four ledgers:
    reserved VA, created handles, mapped handles, valid active rows, with
    M_mapped = valid + active slack + inactive retained and
    M_phys,pool = M_mapped + free handles (M_VA in neither).
  * 0x06B: virtual range and physical handle have separate state machines; a
    request generation is a third axis: a slot handed to a new request keeps
    its address (and maybe its backing) but none of the old rows' validity.
  * 0x06C: the scalar (slot r, token t, head h, lane d) of tensor X_l sits at
    base(X, l) + r R + u with u = (t H_kv d_h + h d_h + d) b, in virtual page
    q = floor(u / G) at offset u mod G; the kernel reads no block table, only a
    request-slot index.
  * 0x06D: pages are mapped before use; all K and V pages of a request frontier
    become visible together.
  * 0x06E: freeing a slot may retain its mappings; a later request reuses the
    capacity, never the rows; under pressure an inactive slot's highest page
    bundle is unmapped and mapped at an active request's frontier.
  * 0x0BJ: page groups are not kernel blocks: N_G = ceil(T / P_G) groups, waste
    W_G = N_G G - T B_row.

``base(X, l)``: tensors are ordered K_0, V_0, K_1, V_1, ... (index 2l + kind),
each B R bytes, so base(V_1) = 3 B R as in the pages' fixture.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .attention import attention_rows


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass(frozen=True)
class Geometry:
    """The reservation of one worker (0x06A)."""

    layers: int        # L
    slots: int         # B
    max_tokens: int    # T_max
    kv_heads: int      # H_kv
    head_dim: int      # d_h
    scalar_bytes: int  # b
    page_bytes: int    # G

    @property
    def row_bytes(self) -> int:
        return self.kv_heads * self.head_dim * self.scalar_bytes

    @property
    def tokens_per_page(self) -> int:
        if self.page_bytes % self.row_bytes:
            raise ValueError("page size is not a whole number of rows")
        return self.page_bytes // self.row_bytes

    @property
    def slot_bytes(self) -> int:            # R
        return self.page_bytes * ceil_div(self.max_tokens * self.row_bytes, self.page_bytes)

    @property
    def pages_per_slot(self) -> int:
        return self.slot_bytes // self.page_bytes

    @property
    def reserved_bytes(self) -> int:        # M_VA
        return 2 * self.layers * self.slots * self.slot_bytes

    @property
    def page_bundle_bytes(self) -> int:
        return 2 * self.layers * self.page_bytes

    def tensor_base(self, kind: str, layer: int) -> int:
        idx = 2 * layer + (0 if kind == "K" else 1)
        return idx * self.slots * self.slot_bytes

    def address(self, kind: str, layer: int, slot: int, t: int, h: int, lane: int):
        """(A_VA, u, q, delta) of one scalar, row-major [t][h][d] (0x06C)."""
        if not (0 <= t < self.max_tokens and 0 <= h < self.kv_heads and 0 <= lane < self.head_dim):
            raise ValueError("coordinate out of range")
        u = (t * self.kv_heads * self.head_dim + h * self.head_dim + lane) * self.scalar_bytes
        q, delta = divmod(u, self.page_bytes)
        return self.tensor_base(kind, layer) + slot * self.slot_bytes + u, u, q, delta

    def pages_for(self, tokens: int) -> int:
        """Pages of one tensor a slot needs for its first ``tokens`` rows."""
        return ceil_div(tokens * self.row_bytes, self.page_bytes)


def page_group_staircase(T: int, row_bytes: int, page_bytes: int) -> Tuple[int, int]:
    """(N_G, W_G): page groups for T rows and the bytes they leave unused (0x0BJ)."""
    if page_bytes % row_bytes:
        raise ValueError("page size is not a whole number of rows")
    n = ceil_div(T, page_bytes // row_bytes)
    return n, n * page_bytes - T * row_bytes


class MappingFailure(RuntimeError):
    """No free handle and no inactive slot page to reclaim: nothing changed."""


@dataclass
class Slot:
    active: bool = False
    generation: int = 0
    valid_tokens: int = 0
    mapped_pages: int = 0      # frontier: pages [0, mapped_pages) of every tensor


class Arena:
    """The runtime state machines of 0x06B-0x06E over one reservation.

    A page bundle (page q of a slot in all 2L tensors) takes 2L handles.
    ``ensure`` maps the missing bundles of a slot in page order, taking free
    handles first and then reclaiming the highest bundle of an inactive slot
    (lowest slot index first); if neither is possible it returns every handle
    it took and raises, leaving the state unchanged.
    """

    def __init__(self, geom: Geometry, num_handles: int):
        self.g = geom
        self.free_handles = list(range(num_handles))
        self.num_handles = num_handles
        self.slots = [Slot() for _ in range(geom.slots)]
        self.mapping: Dict[Tuple[int, int], List[int]] = {}   # (slot, q) -> 2L handles
        self.maps = 0
        self.unmaps = 0

    # -- lifecycle -----------------------------------------------------------------
    def allocate(self, slot: int) -> int:
        """Bind slot to a new request generation: no row is valid (0x06B, 0x06E)."""
        s = self.slots[slot]
        if s.active:
            raise ValueError("slot already active")
        s.active = True
        s.generation += 1
        s.valid_tokens = 0
        return s.generation

    def free(self, slot: int, retain: bool = True) -> None:
        s = self.slots[slot]
        if not s.active:
            raise ValueError("slot not active")
        s.active = False
        s.valid_tokens = 0
        if not retain:
            while s.mapped_pages:
                self._unmap_top(slot)

    def ensure(self, slot: int, tokens: int) -> int:
        """Map pages so that ``tokens`` rows of the slot are backed; returns the
        number of bundles mapped by this call.  All or nothing: on failure the
        whole state is restored (no half-published frontier, 0x06D)."""
        s = self.slots[slot]
        if not s.active:
            raise ValueError("slot not active")
        if tokens > self.g.max_tokens:
            raise ValueError("beyond the reservation")
        need = self.g.pages_for(tokens)
        per = 2 * self.g.layers
        saved = (list(self.free_handles), dict(self.mapping),
                 [sl.mapped_pages for sl in self.slots], self.maps, self.unmaps)
        mapped = 0
        for q in range(s.mapped_pages, need):
            handles = self._take(per, slot)
            if handles is None:
                self.free_handles, self.mapping = saved[0], saved[1]
                for sl, mp in zip(self.slots, saved[2]):
                    sl.mapped_pages = mp
                self.maps, self.unmaps = saved[3], saved[4]
                raise MappingFailure(f"slot {slot}: no handles for page {q}")
            self.mapping[(slot, q)] = handles
            mapped += 1
        s.mapped_pages = max(s.mapped_pages, need)
        self.maps += mapped
        return mapped

    def commit(self, slot: int, tokens: int) -> None:
        """Rows [0, tokens) of the slot hold this generation's K/V (after the
        writes); only mapped rows can be committed (map before use)."""
        s = self.slots[slot]
        if tokens > self.capacity(slot):
            raise ValueError("rows beyond the mapped frontier")
        s.valid_tokens = tokens

    def capacity(self, slot: int) -> int:
        """Rows backed by the slot's mapped frontier."""
        return min(self.g.max_tokens, self.slots[slot].mapped_pages * self.g.page_bytes // self.g.row_bytes)

    # -- handles ---------------------------------------------------------------------
    def _take(self, n: int, slot: int) -> Optional[List[int]]:
        while len(self.free_handles) < n:
            victim = next((v for v, s in enumerate(self.slots)
                           if v != slot and not s.active and s.mapped_pages), None)
            if victim is None:
                return None
            self._unmap_top(victim)
        hs, self.free_handles = self.free_handles[:n], self.free_handles[n:]
        return hs

    def _unmap_top(self, slot: int) -> None:
        s = self.slots[slot]
        q = s.mapped_pages - 1
        self.free_handles.extend(self.mapping.pop((slot, q)))
        s.mapped_pages = q
        self.unmaps += 1

    # -- ledgers (0x06A) -----------------------------------------------------------
    def ledgers(self) -> Dict[str, int]:
        g = self.g
        per_page = 2 * g.layers * g.page_bytes
        mapped = len(self.mapping) * per_page
        valid = sum(2 * g.layers * s.valid_tokens * g.row_bytes for s in self.slots if s.active)
        active_mapped = sum(s.mapped_pages * per_page for s in self.slots if s.active)
        inactive = sum(s.mapped_pages * per_page for s in self.slots if not s.active)
        return {"va": g.reserved_bytes, "phys_pool": self.num_handles * g.page_bytes,
                "mapped": mapped, "active_valid": valid, "active_slack": active_mapped - valid,
                "inactive_retained": inactive, "free_handles": len(self.free_handles) * g.page_bytes}

    def check(self) -> None:
        led = self.ledgers()
        if led["mapped"] != led["active_valid"] + led["active_slack"] + led["inactive_retained"]:
            raise AssertionError("mapped backing does not reconcile")
        if led["phys_pool"] != led["mapped"] + led["free_handles"]:
            raise AssertionError("physical pool does not reconcile")
        seen = set(self.free_handles)
        for hs in self.mapping.values():
            if seen & set(hs):
                raise AssertionError("a handle is both free and mapped, or mapped twice")
            seen |= set(hs)
        if len(seen) != self.num_handles:
            raise AssertionError("a handle is lost")
        for v, s in enumerate(self.slots):
            for q in range(s.mapped_pages):
                if (v, q) not in self.mapping:
                    raise AssertionError("frontier with a hole")


def contiguous_decode(rows_k: Sequence[np.ndarray], rows_v: Sequence[np.ndarray],
                      q: np.ndarray, slot_index: Sequence[int], seq_lens: Sequence[int],
                      scale: float, group: int):
    """Decode with a request-slot index and no block table (0x06C): row i of
    the batch reads rows [0, T_i) of slot slot_index[i].

    rows_k[s], rows_v[s]: binary64 [T_max, H_kv, d] contents of slot s (rows
    past the valid length never read); q: binary64 [B, H_q, d].  Returns
    (out [B, H_q, d], lse [B, H_q])."""
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for i in range(B):
        s, T = int(slot_index[i]), int(seq_lens[i])
        for h in range(Hq // group):
            K = rows_k[s][:T, h]
            V = rows_v[s][:T, h]
            O, L = attention_rows(q[i, h * group:(h + 1) * group], K, V, scale)
            out[i, h * group:(h + 1) * group] = O
            lse[i, h * group:(h + 1) * group] = L
    return out, lse
