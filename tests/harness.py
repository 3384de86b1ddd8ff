"""Test harness: run a workload script through the oracle allocator, then replay
the resulting physical trace on the oracle's bit pool and on the GPU library.

Only tests and ``__graft_entry__.smoke()`` use this module (it imports the
oracle).  The GPU side receives exactly the same slots, copy pairs, tables,
lengths and scalar bits as the oracle; nothing flows back from the GPU into the
oracle.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

import workloads as wl
from oracle.allocator import BlockAllocator
from oracle.pool import BitPool


@dataclass
class Executed:
    workload: wl.Workload
    alloc: BlockAllocator
    ops: List[Tuple]            # ("append", slots, row_lo, row_hi) | ("copy", src, dst)
    tables: np.ndarray          # int32 [B, max_blocks], -1 padded
    seq_lens: np.ndarray        # int32 [B]
    n_writes: int


def execute(w: wl.Workload, max_blocks: int = None) -> Executed:
    """Run the script on a fresh oracle allocator whose FIFO starts in the
    workload's seeded order; group the trace into append / copy calls."""
    a = BlockAllocator(w.shape.num_blocks, w.shape.block_size, free_order=wl.fifo_order(w))
    for act in w.actions:
        kind = act[0]
        if kind == "new":
            a.new_request()
        elif kind == "prefill":
            a.prefill(act[1], act[2])
        elif kind == "append":
            a.append(act[1])
        elif kind == "fork":
            a.fork(act[1])
        elif kind == "release":
            a.release(act[1])
        else:
            raise ValueError(act)
    a.check_invariants()
    ops = group_trace(a.trace)
    n_writes = sum(1 for op in a.trace if op[0] == "write")
    lens = np.array([a.length(r) for r in w.decode], dtype=np.int32)
    widths = [len(a.table(r)) for r in w.decode]
    mb = max_blocks or max(widths)
    tables = np.full((len(w.decode), mb), -1, dtype=np.int32)
    for i, r in enumerate(w.decode):
        t = a.table(r)
        tables[i, :len(t)] = t
    return Executed(w, a, ops, tables, lens, n_writes)


def group_trace(trace) -> List[Tuple]:
    """Consecutive writes become one append call (split at a repeated slot);
    consecutive copies become one copy call (split at any conflict)."""
    ops: List[Tuple] = []
    w = 0
    cur_slots: List[int] = []
    cur_lo = 0
    seen = set()
    pairs_src: List[int] = []
    pairs_dst: List[int] = []
    busy = set()

    def flush_writes():
        nonlocal cur_slots, seen, cur_lo
        if cur_slots:
            ops.append(("append", np.array(cur_slots, dtype=np.int64), cur_lo, cur_lo + len(cur_slots)))
        cur_slots, seen = [], set()
        cur_lo = w

    def flush_copies():
        nonlocal pairs_src, pairs_dst, busy
        if pairs_src:
            ops.append(("copy", np.array(pairs_src, dtype=np.int32), np.array(pairs_dst, dtype=np.int32)))
        pairs_src, pairs_dst, busy = [], [], set()

    for op in trace:
        if op[0] == "write":
            flush_copies()
            if op[3] in seen:
                flush_writes()
            if not cur_slots:
                cur_lo = w
            cur_slots.append(op[3])
            seen.add(op[3])
            w += 1
        else:
            flush_writes()
            s, d = op[1], op[2]
            if s in busy or d in busy:
                flush_copies()
            pairs_src.append(s)
            pairs_dst.append(d)
            busy.update((s, d))
    flush_writes()
    flush_copies()
    return ops


def oracle_pool(ex: Executed, k_rows: np.ndarray, v_rows: np.ndarray) -> BitPool:
    k0, v0 = wl.pool_poison(ex.workload)
    pool = BitPool(k0, v0, ex.workload.shape.dtype)
    for op in ex.ops:
        if op[0] == "append":
            pool.kv_append(op[1], k_rows[op[2]:op[3]], v_rows[op[2]:op[3]])
        else:
            pool.block_copy(op[1], op[2])
    return pool


# ---------------------------------------------------------------------------
# GPU side (torch tensors; the library does the work)
# ---------------------------------------------------------------------------
def to_device(bits: np.ndarray, dtype: str, device):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int32)).view(torch.float32).to(device)


def to_bits(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def gpu_pool(ex: Executed, device):
    import block_table_attention_amd as pba

    k0, v0 = wl.pool_poison(ex.workload)
    dt = ex.workload.shape.dtype
    return pba.KVPool(to_device(k0, dt, device), to_device(v0, dt, device))


def gpu_replay(ex: Executed, pool, k_rows_dev, v_rows_dev, stream=None):
    """Issue the grouped trace on the GPU: every op is a library call, in order."""
    import torch
    import block_table_attention_amd as pba

    dev = pool.k.device
    for op in ex.ops:
        if op[0] == "append":
            slots = torch.from_numpy(op[1]).to(dev)
            pba.kv_append(pool, slots, k_rows_dev[op[2]:op[3]], v_rows_dev[op[2]:op[3]], stream=stream)
        else:
            pba.block_copy(pool, torch.from_numpy(op[1]).to(dev), torch.from_numpy(op[2]).to(dev),
                           stream=stream)


# ---------------------------------------------------------------------------
# Cache groups with a layer axis
# ---------------------------------------------------------------------------
@dataclass
class BundleExecuted:
    workload: wl.BundleWorkload
    alloc: object               # oracle.bundles.BundleAllocator
    ops: List[Tuple]            # ("append", [slots per group], lo, hi) | ("copy", [(src, dst) per group])
    tables: List[np.ndarray]    # per group: int32 [B, max_blocks_g], -1 padded
    seq_lens: np.ndarray        # int32 [B]
    n_writes: int


def execute_bundle(w: wl.BundleWorkload) -> BundleExecuted:
    """Run the script on the oracle's bundle allocator (every group's FIFO in
    its seeded order) and group its trace into bundle append / copy calls."""
    from oracle.bundles import BundleAllocator

    G = len(w.groups)
    a = BundleAllocator([g.num_blocks for g in w.groups], [g.block_size for g in w.groups],
                        free_orders=[o.tolist() for o in wl.bundle_fifo_orders(w)])
    for act in w.actions:
        kind = act[0]
        if kind == "new":
            a.new_request()
        elif kind == "prefill":
            a.prefill(act[1], act[2])
        elif kind == "append":
            a.append(act[1])
        elif kind == "fork":
            a.fork(act[1])
        elif kind == "release":
            a.release(act[1])
        else:
            raise ValueError(act)
    a.check_invariants()
    ops: List[Tuple] = []
    w_idx = 0
    cur: List[List[int]] = [[] for _ in range(G)]
    seen = [set() for _ in range(G)]
    lo = 0
    pairs: List[List[Tuple[int, int]]] = [[] for _ in range(G)]
    busy = [set() for _ in range(G)]

    def flush_writes():
        nonlocal cur, seen, lo
        if cur[0]:
            ops.append(("append", [np.array(c, dtype=np.int64) for c in cur], lo, lo + len(cur[0])))
        cur = [[] for _ in range(G)]
        seen = [set() for _ in range(G)]
        lo = w_idx

    def flush_copies():
        nonlocal pairs, busy
        if any(pairs):
            ops.append(("copy", [(np.array([s for s, _ in p], dtype=np.int32),
                                  np.array([d for _, d in p], dtype=np.int32)) for p in pairs]))
        pairs = [[] for _ in range(G)]
        busy = [set() for _ in range(G)]

    tr = a.trace
    i = 0
    while i < len(tr):
        if tr[i][0] == "write":
            flush_copies()
            slots = [tr[i + g][4] for g in range(G)]       # one write per group, in group order
            assert all(tr[i + g][0] == "write" and tr[i + g][1] == g for g in range(G))
            if any(slots[g] in seen[g] for g in range(G)):
                flush_writes()
            if not cur[0]:
                lo = w_idx
            for g in range(G):
                cur[g].append(slots[g])
                seen[g].add(slots[g])
            w_idx += 1
            i += G
        else:
            flush_writes()
            _, g, s, d = tr[i]
            if s in busy[g] or d in busy[g]:
                flush_copies()
            pairs[g].append((s, d))
            busy[g].update((s, d))
            i += 1
    flush_writes()
    flush_copies()
    lens = np.array([a.lengths[r] for r in w.decode], dtype=np.int32)
    tables = []
    for g in range(G):
        mb = max(len(a.table(r, g)) for r in w.decode)
        t = np.full((len(w.decode), mb), -1, dtype=np.int32)
        for j, r in enumerate(w.decode):
            row = a.table(r, g)
            t[j, :len(row)] = row
        tables.append(t)
    return BundleExecuted(w, a, ops, tables, lens, w_idx)


def bundle_manifests(w: wl.BundleWorkload):
    from oracle import bundles as bd

    out = []
    for gs in w.groups:
        k = bd.LAYER_MAJOR_K if gs.layer_major else bd.BLOCK_MAJOR_K
        v = bd.LAYER_MAJOR_V if gs.layer_major else bd.BLOCK_MAJOR_V
        out.append(bd.GroupManifest(gs.layers, gs.num_blocks, gs.block_size, w.num_kv_heads,
                                    w.head_dim, w.dtype, k, v))
    return out


def oracle_bundle_pools(ex: BundleExecuted, rows):
    """Layered oracle pools of every group after the grouped ops; rows[g] =
    (k, v) bits [n_writes, L_g, H, d]."""
    from oracle import bundles as bd

    w = ex.workload
    pools = []
    for g, m in enumerate(bundle_manifests(w)):
        k0, v0 = wl.bundle_poison(w, g)
        pools.append(bd.LayeredPool(m, k0, v0))
    for op in ex.ops:
        if op[0] == "append":
            bd.bundle_append(pools, [s.tolist() for s in op[1]],
                             [r[0][op[2]:op[3]] for r in rows], [r[1][op[2]:op[3]] for r in rows])
        else:
            bd.bundle_copy(pools, [list(zip(s.tolist(), d.tolist())) for s, d in op[1]])
    return pools


def gpu_bundle_groups(w: wl.BundleWorkload, device):
    import block_table_attention_amd as pba

    groups = []
    for g, gs in enumerate(w.groups):
        k0, v0 = wl.bundle_poison(w, g)
        lead = (gs.layers, gs.num_blocks) if gs.layer_major else (gs.num_blocks, gs.layers)
        k = to_device(k0, w.dtype, device).view(lead + (w.num_kv_heads, gs.block_size, w.head_dim))
        v = to_device(v0, w.dtype, device).view(lead + (w.num_kv_heads, w.head_dim, gs.block_size))
        groups.append(pba.KVGroup(k, v, gs.layer_major))
    return groups


def gpu_bundle_replay(ex: BundleExecuted, groups, rows_dev, per_layer: bool = False, stream=None):
    """Issue the grouped ops on the GPU: one bundle call per op, or (per_layer)
    the single-layer calls of every layer of every group."""
    import torch
    import block_table_attention_amd as pba

    dev = groups[0].k.device
    for op in ex.ops:
        if op[0] == "append":
            slots = [torch.from_numpy(s).to(dev) for s in op[1]]
            ks = [r[0][op[2]:op[3]] for r in rows_dev]
            vs = [r[1][op[2]:op[3]] for r in rows_dev]
            if not per_layer:
                pba.kv_append_bundle(groups, slots, ks, vs, stream=stream)
                continue
            for g, grp in enumerate(groups):
                for l in range(grp.num_layers):
                    pba.kv_append(grp.layer(l), slots[g], ks[g][:, l].contiguous(),
                                  vs[g][:, l].contiguous(), stream=stream)
        else:
            src = [torch.from_numpy(s).to(dev) for s, _ in op[1]]
            dst = [torch.from_numpy(d).to(dev) for _, d in op[1]]
            if not per_layer:
                pba.block_copy_bundle(groups, src, dst, stream=stream)
                continue
            for g, grp in enumerate(groups):
                if src[g].numel():
                    for l in range(grp.num_layers):
                        pba.block_copy(grp.layer(l), src[g], dst[g], stream=stream)
