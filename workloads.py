"""Seeded synthetic workloads shared by the tests, ``smoke()`` and ``bench.py``.

This module holds only random draws and shapes: request lengths, the starting
order of the free FIFO, K/V/q scalar bits, NaN-poisoned initial pool bits, and
each workload's script of request actions (new request, prefill, fork,
release, one-token append).  It contains no attention arithmetic, no address
translation and no allocator: executing a script (turning actions into block
tables, slot ids and copy pairs) is the caller's job.

Scalar draws: N(0, 1) binary32 from a seeded ``torch.Generator`` on the CPU,
rounded to bfloat16 by round-to-nearest-even where the workload is bf16.  The
stored bits are what everybody reads.  Structure draws use
``numpy.random.default_rng``.  Seeds are ``20261202 + 100 * workload_index +
rep`` with a small per-component offset.

Workloads (sizes follow the pages' workload descriptions; there is no public
dataset for this path, and these synthetic generators stand in for the pages'
short chats, shared system prompts, parallel samples and long documents):

  tiny           1 request x 35 tokens, P=16, 1 q-head / 1 kv-head, d=64, f32,
                 32-block pool
  batch32        32 requests, T_r ~ U{64..2048}, then one appended token each,
                 P=16, 32q/8kv, d=128, bf16, 8192-block pool
  shared_prefix  one 2000-token prefix forked to 64 requests (the parent is
                 released), private suffixes U{12..700}, then every request is
                 forked once more and each sibling appends one token (the
                 divergent append into a shared tail), 32q/8kv, d=128, bf16,
                 P=16, 8192-block pool
  lognormal      128 requests, lognormal lengths with median 100 and max 8192,
                 P in {16, 64, 256}, 32q/8kv, d=128, bf16, pool of
                 ceil(1.25 * sum ceil(T_r/P)) blocks
  long16k        8 requests x 16,384 tokens at decode time (16,383 prefilled +
                 1 appended), P=64, 64q/8kv, d=128, bf16, 4096-block pool
  long64k        1 request x 65,536 tokens (65,535 + 1), otherwise as long16k
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np

SEED_BASE = 20261202
WORKLOAD_INDEX = {"tiny": 1, "batch32": 2, "shared_prefix": 3, "lognormal": 4,
                  "long16k": 5, "long64k": 5, "layers32": 6, "bundle": 7}

# Per-component seed offsets.
_K, _V, _Q, _POISON, _STRUCT, _ORDER = 1, 2, 3, 4, 5, 6


def seed_for(name: str, rep: int = 0) -> int:
    return SEED_BASE + 100 * WORKLOAD_INDEX[name] + rep


@dataclass(frozen=True)
class Shape:
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str          # "bf16" | "f32"
    num_blocks: int


@dataclass
class Workload:
    """A script of request actions plus everything needed to draw its scalars.

    actions: ("new",) | ("prefill", rid, n) | ("fork", rid) | ("release", rid)
             | ("append", rid); request ids are numbered 0, 1, 2 ... in the
             order "new" and "fork" create them.
    decode:  request ids of the decode batch, in batch order.
    """

    name: str
    shape: Shape
    seed: int
    actions: List[Tuple] = field(default_factory=list)
    decode: List[int] = field(default_factory=list)

    def n_writes(self) -> int:
        return sum(a[2] if a[0] == "prefill" else 1 for a in self.actions
                   if a[0] in ("prefill", "append"))


# ---------------------------------------------------------------------------
# Scalar draws
# ---------------------------------------------------------------------------
def normal_bits(seed: int, shape: Sequence[int], dtype: str) -> np.ndarray:
    """N(0,1) binary32 draws; bf16 by round-to-nearest-even.  Returns raw bits."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32)
    if dtype == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f32":
        return x.view(torch.int32).numpy().view(np.uint32)
    raise ValueError(dtype)


def poison_bits(seed: int, shape: Sequence[int], dtype: str) -> np.ndarray:
    """Quiet/signalling NaN bit patterns with random sign and nonzero payload.

    A pool filled with these makes any read of a row that was never written
    (padding, tail, recycled garbage) show up as NaN in the result, and checks
    that bit copies keep NaN payloads.
    """
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    if dtype == "bf16":
        mant = rng.integers(1, 1 << 7, size=n, dtype=np.uint16)
        sign = rng.integers(0, 2, size=n, dtype=np.uint16) << np.uint16(15)
        return (sign | np.uint16(0x7F80) | mant).reshape(shape)
    if dtype == "f32":
        mant = rng.integers(1, 1 << 23, size=n, dtype=np.uint32)
        sign = rng.integers(0, 2, size=n, dtype=np.uint32) << np.uint32(31)
        return (sign | np.uint32(0x7F800000) | mant).reshape(shape)
    raise ValueError(dtype)


def free_order(seed: int, num_blocks: int) -> np.ndarray:
    """Starting order of the free FIFO: a seeded permutation of all block ids."""
    return np.random.default_rng(seed).permutation(num_blocks).astype(np.int64)


def uniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on {lo, ..., hi}."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=n).astype(np.int64)


def lognormal_lengths(seed: int, n: int, median: int = 100, max_len: int = 8192) -> np.ndarray:
    """Lognormal lengths with the given median, clipped to [1, max_len].

    sigma puts max_len at the 1 - 1/128 quantile (z = Phi^-1(1 - 1/128)); the
    largest draw is then set to max_len so the batch always holds one request
    of the maximum length.
    """
    z = _normal_quantile(1.0 - 1.0 / 128.0)
    mu = math.log(median)
    sigma = math.log(max_len / median) / z
    rng = np.random.default_rng(seed)
    x = np.exp(mu + sigma * rng.standard_normal(n))
    lengths = np.clip(np.rint(x), 1, max_len).astype(np.int64)
    lengths[int(np.argmax(lengths))] = max_len
    return lengths


def _normal_quantile(p: float) -> float:
    """Inverse standard normal CDF by bisection on math.erf (shape parameter only)."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * (1.0 + math.erf(mid / math.sqrt(2.0))) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# ---------------------------------------------------------------------------
# Workload scripts
# ---------------------------------------------------------------------------
def tiny(rep: int = 0) -> Workload:
    s = seed_for("tiny", rep)
    w = Workload("tiny", Shape(16, 1, 1, 64, "f32", 32), s)
    w.actions = [("new",), ("prefill", 0, 35)]
    w.decode = [0]
    return w


def batch32(rep: int = 0, batch: int = 32, lo: int = 64, hi: int = 2048,
            num_blocks: int = 8192) -> Workload:
    s = seed_for("batch32", rep)
    w = Workload("batch32", Shape(16, 32, 8, 128, "bf16", num_blocks), s)
    lengths = uniform_lengths(s + _STRUCT, batch, lo, hi)
    for r in range(batch):
        w.actions.append(("new",))
        w.actions.append(("prefill", r, int(lengths[r])))
    for r in range(batch):
        w.actions.append(("append", r))
    w.decode = list(range(batch))
    return w


def shared_prefix(rep: int = 0, prefix: int = 2000, children: int = 64,
                  lo: int = 12, hi: int = 700, num_blocks: int = 8192) -> Workload:
    s = seed_for("shared_prefix", rep)
    w = Workload("shared_prefix", Shape(16, 32, 8, 128, "bf16", num_blocks), s)
    suffix = uniform_lengths(s + _STRUCT, children, lo, hi)
    w.actions = [("new",), ("prefill", 0, prefix)]
    kids = list(range(1, children + 1))
    for _ in kids:
        w.actions.append(("fork", 0))
    w.actions.append(("release", 0))
    for i, c in enumerate(kids):
        w.actions.append(("prefill", c, int(suffix[i])))
    sibs = list(range(children + 1, 2 * children + 1))
    for c in kids:
        w.actions.append(("fork", c))
    for sib in sibs:
        w.actions.append(("append", sib))
    w.decode = kids + sibs
    return w


def lognormal(block_size: int, rep: int = 0, batch: int = 128) -> Workload:
    s = seed_for("lognormal", rep)
    lengths = lognormal_lengths(s + _STRUCT, batch)
    n_blocks = int(math.ceil(1.25 * sum(-(-int(T) // block_size) for T in lengths)))
    w = Workload(f"lognormal_p{block_size}", Shape(block_size, 32, 8, 128, "bf16", n_blocks), s)
    for r in range(batch):
        w.actions.append(("new",))
        w.actions.append(("prefill", r, int(lengths[r])))
    w.decode = list(range(batch))
    return w


def long_context(batch: int, context: int, rep: int = 0, num_blocks: int = 4096,
                 block_size: int = 64, num_q_heads: int = 64, num_kv_heads: int = 8,
                 head_dim: int = 128, name: str = None) -> Workload:
    name = name or ("long16k" if batch == 8 else "long64k")
    s = seed_for("long16k", rep)
    w = Workload(name, Shape(block_size, num_q_heads, num_kv_heads, head_dim, "bf16",
                             num_blocks), s)
    for r in range(batch):
        w.actions.append(("new",))
        w.actions.append(("prefill", r, context - 1))
    for r in range(batch):
        w.actions.append(("append", r))
    w.decode = list(range(batch))
    return w


def long16k(rep: int = 0) -> Workload:
    return long_context(8, 16384, rep, name="long16k")


def long64k(rep: int = 0) -> Workload:
    return long_context(1, 65536, rep, name="long64k")


# ---------------------------------------------------------------------------
# Draws bound to a workload
# ---------------------------------------------------------------------------
def kv_rows(w: Workload, n: int, offset: int = 0):
    """K and V bits [n, H_kv, d] for write ops offset .. offset+n-1 of the script.

    Drawn in one piece for the whole script so any prefix of it is stable.
    """
    sh = w.shape
    total = w.n_writes()
    k = normal_bits(w.seed * 16 + _K, (total, sh.num_kv_heads, sh.head_dim), sh.dtype)
    v = normal_bits(w.seed * 16 + _V, (total, sh.num_kv_heads, sh.head_dim), sh.dtype)
    return k[offset:offset + n], v[offset:offset + n]


def q_bits(w: Workload) -> np.ndarray:
    sh = w.shape
    return normal_bits(w.seed * 16 + _Q, (len(w.decode), sh.num_q_heads, sh.head_dim), sh.dtype)


def pool_poison(w: Workload):
    """Initial K pool [NB, H, P, d] and V pool [NB, H, d, P] bits."""
    sh = w.shape
    k = poison_bits(w.seed * 16 + _POISON,
                    (sh.num_blocks, sh.num_kv_heads, sh.block_size, sh.head_dim), sh.dtype)
    v = poison_bits(w.seed * 16 + _POISON + 8,
                    (sh.num_blocks, sh.num_kv_heads, sh.head_dim, sh.block_size), sh.dtype)
    return k, v


def fifo_order(w: Workload) -> np.ndarray:
    return free_order(w.seed * 16 + _ORDER, w.shape.num_blocks)


# ---------------------------------------------------------------------------
# Cache groups with a layer axis
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class GroupShape:
    layers: int
    block_size: int
    num_blocks: int
    layer_major: bool   # K [L, NB, H, P, d]; else block major K [NB, L, H, P, d]


@dataclass
class BundleWorkload:
    """A request script over several cache groups (one block table per group
    and request, one length per request); same action vocabulary as
    ``Workload``."""

    name: str
    groups: List[GroupShape]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    seed: int
    actions: List[Tuple] = field(default_factory=list)
    decode: List[int] = field(default_factory=list)

    def n_writes(self) -> int:
        return sum(a[2] if a[0] == "prefill" else 1 for a in self.actions
                   if a[0] in ("prefill", "append"))

    @property
    def total_layers(self) -> int:
        return sum(g.layers for g in self.groups)


def bundle_rows(w: BundleWorkload, g: int):
    """K and V bits [n_writes, L_g, H_kv, d] of group g, write w = token w."""
    n = w.n_writes()
    shape = (n, w.groups[g].layers, w.num_kv_heads, w.head_dim)
    k = normal_bits(w.seed * 16 + _K + 100 * g, shape, w.dtype)
    v = normal_bits(w.seed * 16 + _V + 100 * g, shape, w.dtype)
    return k, v


def bundle_q_bits(w: BundleWorkload) -> np.ndarray:
    """Decode queries of every model layer: bits [total_layers, B, H_q, d]."""
    return normal_bits(w.seed * 16 + _Q, (w.total_layers, len(w.decode), w.num_q_heads,
                                         w.head_dim), w.dtype)


def bundle_poison(w: BundleWorkload, g: int):
    """Initial K and V bits of group g, flat, in the group's memory order."""
    gs = w.groups[g]
    n = gs.layers * gs.num_blocks * w.num_kv_heads * gs.block_size * w.head_dim
    k = poison_bits(w.seed * 16 + _POISON + 100 * g, (n,), w.dtype)
    v = poison_bits(w.seed * 16 + _POISON + 8 + 100 * g, (n,), w.dtype)
    return k, v


def bundle_fifo_orders(w: BundleWorkload) -> List[np.ndarray]:
    return [free_order(w.seed * 16 + _ORDER + 100 * g, gs.num_blocks)
            for g, gs in enumerate(w.groups)]


def layers32(rep: int = 0, batch: int = 32, forks: int = 8, lo: int = 64,
             hi: int = 2048) -> BundleWorkload:
    """All 32 layers of one tensor-parallel rank of an 8-kv-head, 32-q-head,
    d = 128 model at TP 2 (4 kv heads and 16 q heads per rank), in the pages'
    two cache groups: layers 0-23 (block major) and 24-31 (layer major), both
    with P = 16, bf16.  ``batch`` requests of U[lo, hi] tokens; ``forks`` of
    them are forked, and the step appends one token to every request, so each
    forked pair copies its shared tail bundle first."""
    s = seed_for("layers32", rep)
    lengths = uniform_lengths(s + _STRUCT, batch, lo, hi)
    blocks = sum(-(-(int(T) + 1) // 16) for T in lengths) + forks
    nb = int(math.ceil(1.25 * blocks))
    w = BundleWorkload("layers32", [GroupShape(24, 16, nb, False), GroupShape(8, 16, nb, True)],
                       16, 4, 128, "bf16", s)
    for r in range(batch):
        w.actions.append(("new",))
        w.actions.append(("prefill", r, int(lengths[r]) - 1))
    kids = list(range(batch, batch + forks))
    for i in range(forks):
        w.actions.append(("fork", i))
    for r in list(range(batch)) + kids:
        w.actions.append(("append", r))
    w.decode = list(range(batch)) + kids
    return w
