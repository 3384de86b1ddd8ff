"""Shared-prefix execution reuse over a chunk tree, three ways.

Test infrastructure only (see ``oracle/__init__.py``).

Follows "M5.3 - KV Memory Layout and Exact Reuse":
  * 0x0BA: the legal keys of sequence r are split into disjoint sets, one per
    chunk of its path; each set yields a partial state (valid, m, l, u), and
    the row is recovered by the log-sum-exp merge of those states, never by
    averaging normalised outputs.  An empty set is the identity.
  * 0x0BB: an immutable snapshot holds the queries, the chunks (K/V rows and a
    half-open coverage interval of sequence indices) and each sequence's
    ordered chunk path; sequence r's path contains chunk c exactly when r lies
    in c's coverage.
  * 0x0BC (Hydragen coordinates): every chunk is attended by all the queries it
    covers at once, giving a normalised output and an LSE per covered row;
    the rows are merged in (output, LSE) coordinates.
  * 0x0BD (ChunkAttention coordinates): a chunk-first phase materialises the
    (u, m, l) state of every chunk whose coverage exceeds a threshold, for all
    covered rows; a sequence-first phase walks each path, computes the states
    of the other chunks for that sequence alone, and merges everything.
  * 0x0BE: the K/V rows each schedule loads (monolithic: every logical pair;
    chunked: every chunk once) and the number of materialised partial rows.

All arithmetic is binary64 numpy; queries are [B, G, d_qk], chunk K [T_c, d_qk]
and V [T_c, d_v] (d_v may differ from d_qk, as in the pages' fixture).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

from .attention import PartialState, merge_states, partial_state


@dataclass
class Chunk:
    K: np.ndarray          # [T_c, d_qk]
    V: np.ndarray          # [T_c, d_v]
    begin: int             # coverage: sequences [begin, end)
    end: int


@dataclass
class Snapshot:
    Q: np.ndarray                  # [B, G, d_qk]
    chunks: List[Chunk]
    paths: List[List[int]]         # chunk indices of each sequence, in key order

    def check(self) -> None:
        """The coverage contract of 0x0BB: path membership equals coverage."""
        B = self.Q.shape[0]
        if len(self.paths) != B:
            raise ValueError("one path per sequence")
        for c, ch in enumerate(self.chunks):
            if not 0 <= ch.begin < ch.end <= B:
                raise ValueError(f"chunk {c}: bad coverage [{ch.begin}, {ch.end})")
            if ch.K.shape[0] != ch.V.shape[0]:
                raise ValueError(f"chunk {c}: K and V row counts differ")
            for r in range(B):
                if (ch.begin <= r < ch.end) != (c in self.paths[r]):
                    raise ValueError(f"chunk {c} coverage disagrees with the path of sequence {r}")
        for r, path in enumerate(self.paths):
            if len(set(path)) != len(path):
                raise ValueError(f"sequence {r}: a chunk repeats in its path")


@dataclass
class Result:
    O: np.ndarray          # [B, G, d_v]
    lse: np.ndarray        # [B, G]
    kv_rows_read: int      # K/V rows the schedule loads (0x0BE payload ledger)
    partial_rows: int      # materialised (sequence, chunk) partial states


def _attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Plain softmax attention of the rows of q over (K, V): (O, LSE)."""
    s = (q @ K.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1)
    return (p @ V) / l[:, None], m[:, 0] + np.log(l)


def monolithic(snap: Snapshot, scale: float) -> Result:
    """Reference schedule: concatenate each sequence's path, one attention row."""
    snap.check()
    B, G, _ = snap.Q.shape
    dv = snap.chunks[0].V.shape[1]
    O = np.zeros((B, G, dv))
    lse = np.zeros((B, G))
    rows = 0
    for r, path in enumerate(snap.paths):
        K = np.concatenate([snap.chunks[c].K for c in path])
        V = np.concatenate([snap.chunks[c].V for c in path])
        O[r], lse[r] = _attend(snap.Q[r], K, V, scale)
        rows += K.shape[0]
    return Result(O, lse, rows, 0)


def merge_lse(outputs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Merge normalised outputs by their LSEs (0x0BC): weights exp(LSE_p - max)."""
    L = np.stack(lses)                      # [n, G]
    M = L.max(axis=0)
    w = np.exp(L - M)                       # [n, G]
    tot = w.sum(axis=0)
    O = sum(w[i][:, None] * outputs[i] for i in range(len(outputs))) / tot[:, None]
    return O, M + np.log(tot)


def hydragen(snap: Snapshot, scale: float) -> Result:
    """Every chunk attended once by all the queries it covers; per-sequence
    merge in (output, LSE) coordinates."""
    snap.check()
    B, G, _ = snap.Q.shape
    parts = [[] for _ in range(B)]
    rows = 0
    for ch in snap.chunks:
        qs = snap.Q[ch.begin:ch.end].reshape(-1, snap.Q.shape[2])
        O, L = _attend(qs, ch.K, ch.V, scale)
        rows += ch.K.shape[0]
        n = ch.end - ch.begin
        O = O.reshape(n, G, -1)
        L = L.reshape(n, G)
        for i in range(n):
            parts[ch.begin + i].append((O[i], L[i]))
    dv = snap.chunks[0].V.shape[1]
    out = np.zeros((B, G, dv))
    lse = np.zeros((B, G))
    for r in range(B):
        out[r], lse[r] = merge_lse([p[0] for p in parts[r]], [p[1] for p in parts[r]])
    return Result(out, lse, rows, 0)


def chunk_attention(snap: Snapshot, scale: float, threshold: int) -> Result:
    """Chunk-first for chunks covering more than ``threshold`` sequences,
    sequence-first for the rest; states merged along each path."""
    snap.check()
    B, G, _ = snap.Q.shape
    saved = {}                 # (chunk, sequence) -> PartialState
    rows = 0
    partial_rows = 0
    for c, ch in enumerate(snap.chunks):
        if ch.end - ch.begin <= threshold:
            continue
        rows += ch.K.shape[0]
        for r in range(ch.begin, ch.end):
            saved[(c, r)] = partial_state(snap.Q[r], ch.K, ch.V, scale)
            partial_rows += 1
    dv = snap.chunks[0].V.shape[1]
    out = np.zeros((B, G, dv))
    lse = np.zeros((B, G))
    for r, path in enumerate(snap.paths):
        states: List[PartialState] = []
        for c in path:
            if (c, r) in saved:
                states.append(saved[(c, r)])
            else:
                ch = snap.chunks[c]
                states.append(partial_state(snap.Q[r], ch.K, ch.V, scale))
                rows += ch.K.shape[0]
        out[r], lse[r] = merge_states(states)
    return Result(out, lse, rows, partial_rows)


def random_snapshot(rng: np.random.Generator, tree: Sequence[Tuple[int, Tuple[int, int]]],
                    G: int, d_qk: int, d_v: int) -> Snapshot:
    """A snapshot over a chunk tree given as (rows, (begin, end)) in path order
    (ancestors before descendants); paths follow from the coverages."""
    B = max(e for _, (_, e) in tree)
    chunks = [Chunk(rng.standard_normal((t, d_qk)), rng.standard_normal((t, d_v)), b, e)
              for t, (b, e) in tree]
    paths = [[c for c, ch in enumerate(chunks) if ch.begin <= r < ch.end] for r in range(B)]
    return Snapshot(rng.standard_normal((B, G, d_qk)), chunks, paths)
