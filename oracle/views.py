"""Kernel views of an allocator pool, and compact (ragged) block tables.

Test infrastructure only (see ``oracle/__init__.py``).

Follows "M5.3 - KV Memory Layout and Exact Reuse":
  * 0x0AC: allocator blocks of P_a tokens may be exposed to a kernel as blocks
    of P_k tokens with P_a = q P_k; allocator id a becomes the kernel ids
    a q, ..., a q + q - 1, and kernel block b holds the rows
    [(b mod q) P_k, (b mod q + 1) P_k) of allocator block floor(b / q).  No
    payload moves; only the table grows q-fold.  A kernel block larger than an
    allocator block is rejected.
  * 0x0AB: a dense staging table has B n_max cells; a compact encoding keeps
    each row's n_r = ceil(T_r / P_k) entries back to back with row offsets
    (the prefix sums of n_r), trading padding for offsets and packing work.

The kernel-view gather below reads rows through kernel ids and the split
rule, independently of ``BitPool.gather`` (which reads allocator ids), so the
two can be compared.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .bits import bits_to_f64
from .pool import BitPool


def split_factor(P_a: int, P_k: int) -> int:
    if P_k <= 0 or P_a % P_k:
        raise ValueError("the kernel block size must divide the allocator block size")
    return P_a // P_k


def expand_table(alloc_ids: Sequence[int], P_a: int, P_k: int) -> List[int]:
    """Allocator ids -> kernel ids (each a -> a q .. a q + q - 1)."""
    q = split_factor(P_a, P_k)
    out = []
    for a in alloc_ids:
        out.extend(range(a * q, a * q + q))
    return out


def gather_kernel_view(pool: BitPool, kernel_table: Sequence[int], T: int, head: int,
                       P_k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Logical K, V [T, d] of one head read through kernel block ids."""
    q = split_factor(pool.P, P_k)
    K = np.empty((T, pool.head_dim))
    V = np.empty((T, pool.head_dim))
    for t in range(T):
        b = kernel_table[t // P_k]
        a, i = divmod(b, q)
        row = i * P_k + t % P_k
        K[t] = bits_to_f64(pool.k[a, head, row, :], pool.dtype)
        V[t] = bits_to_f64(pool.v[a, head, :, row], pool.dtype)
    return K, V


def pack_ragged(tables: np.ndarray, seq_lens: Sequence[int], P: int):
    """Dense [B, n_max] table -> (entries [sum n_r], offsets [B + 1])."""
    n = [-(-int(T) // P) for T in seq_lens]
    offsets = np.zeros(len(n) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(n)
    entries = np.concatenate([np.asarray(tables[r][:n[r]], dtype=np.int32) for r in range(len(n))]) \
        if n else np.zeros(0, dtype=np.int32)
    return entries, offsets


def unpack_ragged(entries: np.ndarray, offsets: np.ndarray, r: int) -> np.ndarray:
    return entries[offsets[r]:offsets[r + 1]]
