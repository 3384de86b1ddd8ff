"""Binary64 softmax attention over each request's logical K/V history.

Test infrastructure only (see ``oracle/__init__.py``).

Paging changes where K/V bytes live, never the attention result
("M5.3 - KV Memory Layout and Exact Reuse", 0x00A-0x00B and 0x0A), so the
oracle is the plain definition written out: gather the request-visible rows in
logical order and evaluate

    s_i = (q . k_i) * scale                        (0x0BA; scale = 1/sqrt(d))
    O   = sum_i exp(s_i - m) v_i / sum_i exp(s_i - m),  m = max_i s_i
    LSE = m + ln sum_i exp(s_i - m)

GQA: query head i reads kv head floor(i / G) with G = H_q / H_kv (contiguous
groups; the pages name head expansion without fixing the map).

Partition states follow 0x0BA: a partition p of the key set carries
(valid_p, m_p, l_p, u_p) with l_p = sum exp(s - m_p) and u_p = sum exp(s - m_p) v;
its LSE is m_p + ln l_p and its output u_p / l_p.  The merge rescales every
valid state to the common maximum and adds; an empty partition is the identity
and is skipped before any exp(-inf - (-inf)).  Normalised partial outputs are
never averaged.  Partition count for a row of T keys in P_part-key partitions
is ceil(T / P_part) (0x0A).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

from .pool import BitPool
from .bits import bits_to_f64


def attention_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """q [G, d], K [T, d], V [T, d] (binary64) -> O [G, d], LSE [G]."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    if K.shape[0] == 0:
        raise ValueError("a decode row needs at least one visible key")
    s = (q @ K.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1)
    O = (p @ V) / l[:, None]
    return O, m[:, 0] + np.log(l)


def paged_decode(pool: BitPool, q_bits: np.ndarray, tables: Sequence[Sequence[int]],
                 seq_lens: Sequence[int], scale: float,
                 rows: Sequence[Tuple[int, int]] = None):
    """Decode every (request, kv head) pair, or only those listed in ``rows``.

    q_bits: [B, H_q, d] bits of the pool dtype.  Returns (out [B, H_q, d],
    lse [B, H_q]) in binary64; entries of pairs not computed are NaN.
    """
    B, Hq, d = q_bits.shape
    Hkv = pool.kv_heads
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    q = bits_to_f64(q_bits, pool.dtype)
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    pairs = rows if rows is not None else [(r, h) for r in range(B) for h in range(Hkv)]
    for r, h in pairs:
        K, V = pool.gather(tables[r], int(seq_lens[r]), h)
        O, L = attention_rows(q[r, h * G:(h + 1) * G], K, V, scale)
        out[r, h * G:(h + 1) * G] = O
        lse[r, h * G:(h + 1) * G] = L
    return out, lse


@dataclass
class PartialState:
    valid: int          # number of keys in the partition
    m: np.ndarray       # [G] running maximum score
    l: np.ndarray       # [G] sum of exp(s - m)
    u: np.ndarray       # [G, d] sum of exp(s - m) v


def partial_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> PartialState:
    q = np.atleast_2d(q)
    G, d = q.shape
    if K.shape[0] == 0:
        return PartialState(0, np.full(G, -np.inf), np.zeros(G), np.zeros((G, d)))
    s = (q @ K.T) * scale
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return PartialState(K.shape[0], m, p.sum(axis=1), p @ V)


def merge_states(states: List[PartialState]):
    """Log-sum-exp merge of partition states -> (O [G, d], LSE [G])."""
    live = [s for s in states if s.valid > 0]
    if not live:
        raise ValueError("no valid partition: the row has no visible key")
    M = np.max(np.stack([s.m for s in live]), axis=0)
    l = np.zeros_like(M)
    u = np.zeros_like(live[0].u)
    for s in live:
        w = np.exp(s.m - M)
        l = l + w * s.l
        u = u + w[:, None] * s.u
    return u / l[:, None], M + np.log(l)


def num_partitions(T: int, part_tokens: int) -> int:
    return -(-T // part_tokens)


def partitioned_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                          part_tokens: int):
    """Split the keys into ceil(T / P_part) consecutive partitions and merge."""
    T = K.shape[0]
    states = [partial_state(q, K[a:a + part_tokens], V[a:a + part_tokens], scale)
              for a in range(0, T, part_tokens)]
    return merge_states(states)
