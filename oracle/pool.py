"""The K/V pool as raw scalar bits; appends and block copies are bit copies.

Test infrastructure only (see ``oracle/__init__.py``).

Layout (same as the library's documented pool):
  K bits: [num_blocks, H_kv, P, d]   (block, head, in-block token, dim)
  V bits: [num_blocks, H_kv, d, P]   (block, head, dim, in-block token)

``kv_append`` writes row i at slot s_i: block s_i div P, offset s_i mod P
("M5.3", 0x03C-0x03D); a negative slot is skipped.  ``block_copy`` copies whole
physical blocks, K and V, every head and row ("M5.3", 0x04C; "7. Memory
Management and Local Model State", "What branching actually costs").
``gather`` returns the request-visible rows of one head in logical order: full
blocks of P rows and a last block of T mod P rows (P when that is 0), never the
padding or stale rows beyond T ("M5.3", 0x03G, 0x0A, 0x0AC).
"""
from __future__ import annotations

import hashlib
from typing import Iterable, Sequence, Tuple

import numpy as np

from .bits import BITS_DTYPE, bits_to_f64


class BitPool:
    def __init__(self, k_bits: np.ndarray, v_bits: np.ndarray, dtype: str):
        if k_bits.ndim != 4 or v_bits.ndim != 4:
            raise ValueError("pool arrays must be rank 4")
        nb, h, p, d = k_bits.shape
        if v_bits.shape != (nb, h, d, p):
            raise ValueError("V pool must be [num_blocks, H_kv, d, P]")
        self.dtype = dtype
        self.k = np.array(k_bits, dtype=BITS_DTYPE[dtype], copy=True)
        self.v = np.array(v_bits, dtype=BITS_DTYPE[dtype], copy=True)
        self.num_blocks, self.kv_heads, self.P, self.head_dim = nb, h, p, d

    def kv_append(self, slots: Sequence[int], k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        """k_rows, v_rows: bits [n, H_kv, d]."""
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        live = slots[keep]
        if len(np.unique(live)) != len(live):
            raise ValueError("duplicate slot in one append")
        if live.size and (live.max() >= self.num_blocks * self.P):
            raise ValueError("slot outside the pool")
        blk, off = np.divmod(live, self.P)
        self.k[blk, :, off, :] = np.asarray(k_rows)[keep]
        # V tile is [d, P]: the row lands in column ``off`` of every dim.
        self.v[blk, :, :, off] = np.asarray(v_rows)[keep]

    def block_copy(self, src: Sequence[int], dst: Sequence[int]) -> None:
        src = np.asarray(src, dtype=np.int64)
        dst = np.asarray(dst, dtype=np.int64)
        if len(np.unique(dst)) != len(dst) or set(src.tolist()) & set(dst.tolist()):
            raise ValueError("overlapping copy pairs")
        self.k[dst] = self.k[src]
        self.v[dst] = self.v[src]

    def gather(self, table: Sequence[int], T: int, head: int) -> Tuple[np.ndarray, np.ndarray]:
        """Logical K [T, d] and V [T, d] of one head, widened to binary64."""
        P = self.P
        n = -(-T // P)
        ks, vs = [], []
        for j in range(n):
            rows = P if j < n - 1 else T - (n - 1) * P
            b = table[j]
            ks.append(self.k[b, head, :rows, :])
            vs.append(self.v[b, head, :, :rows].T)
        if n == 0:
            d = self.head_dim
            return np.zeros((0, d)), np.zeros((0, d))
        K = bits_to_f64(np.concatenate(ks, axis=0), self.dtype)
        V = bits_to_f64(np.concatenate(vs, axis=0), self.dtype)
        return K, V

    def digest(self) -> str:
        h = hashlib.sha256()
        h.update(np.ascontiguousarray(self.k).tobytes())
        h.update(np.ascontiguousarray(self.v).tobytes())
        return h.hexdigest()


def replay(pool: BitPool, trace: Iterable[Tuple], k_rows: np.ndarray, v_rows: np.ndarray) -> None:
    """Apply an allocator trace in order; write op number w takes row w."""
    w = 0
    for op in trace:
        if op[0] == "copy":
            pool.block_copy([op[1]], [op[2]])
        elif op[0] == "write":
            pool.kv_append([op[3]], k_rows[w:w + 1], v_rows[w:w + 1])
            w += 1
        else:
            raise ValueError(op)
