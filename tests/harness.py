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
