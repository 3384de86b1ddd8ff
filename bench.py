#!/usr/bin/env python3
"""Benchmark: one decode step of paged attention on one MI355X.

A step is one pass of the whole hot path over the decode batch:
  block_copy of the step's copy-on-write pairs, kv_append of the step's new
  tokens (the trailing one-token appends of the workload's script), and
  paged_decode of one query row per request of the batch.  When every new
  token is its row's last position in a block only that row reads, the
  appends ride in the decode call (paged_decode_append, or
  paged_decode_shared_append under a shared-prefix plan); --step separate
  keeps kv_append as a launch of its own.

Default workload: long16k -- 8 requests x 16,384 tokens of context at decode
(16,383 prefilled + 1 appended per step), block size 64, 64 q-heads / 8
kv-heads (GQA 8), head_dim 128, bf16 K/V, pool of 4096 blocks (1 GiB).  The
other workloads (--workload, or --sweep for all of them) follow the same step
on their own scripts.  All inputs are seeded synthetic data, and everything
the step reads is resident in HBM before timing starts.  Block placement comes
from the package's caller-side BlockManager run over the workload's script
from its seeded free-FIFO order.

Prints one JSON line per workload: metric, value (unique K/V bytes the decode
must read, per second of whole steps), step time, query rows/s, the roofline of
the decode kernel (its average launch time over a back-to-back burst, timed
with HIP events on its stream, against HBM peak), and cpu_baseline (the CPU
oracle timed on a bounded sample of the same workload; single-workload runs
only).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOADS = ["long16k", "long64k", "batch32", "shared_prefix", "lognormal_p16",
             "lognormal_p64", "lognormal_p256", "tiny", "layers32"]
BUNDLE_WORKLOADS = {"layers32"}


_SCRUB = None


def cold_launch_ms(torch, fn, stream, reps):
    """(warm, cold) median duration of one launch of fn, each between its own
    pair of HIP events on `stream`; cold launches follow a 1 GiB read that
    evicts the decode's rows from L2 and the 256 MB memory-side cache without
    leaving dirty lines behind (a write scrub would make the decode pay for
    their write-back)."""
    global _SCRUB
    if _SCRUB is None:
        src = torch.ones(1 << 28, dtype=torch.float32, device=stream.device)
        sink = torch.empty(1, dtype=torch.float32, device=stream.device)
        for _ in range(2):
            torch.sum(src, dim=0, keepdim=True, out=sink)
        torch.cuda.synchronize()
        _SCRUB = (src, sink)
    src, sink = _SCRUB
    out = []
    for cold in (False, True):
        evs = []
        for _ in range(reps):
            if cold:
                torch.sum(src, dim=0, keepdim=True, out=sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        out.append(float(np.median([a.elapsed_time(b) for a, b in evs])))
    return out[0], out[1]


AUTO = -2      # --partition-tokens auto: the caller's choice from the batch's lengths
BALANCED = -1  # the library's balanced decomposition (PBA_PARTITIONS_BALANCED)


def _partition_arg(v: str) -> int:
    if v == "auto":
        return AUTO
    if v == "balanced":
        return BALANCED
    return int(v)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long16k", choices=WORKLOADS)
    ap.add_argument("--sweep", action="store_true",
                    help="every workload in turn, one JSON line each (no cpu_baseline)")
    ap.add_argument("--partition-tokens", type=_partition_arg, default=AUTO,
                    help="decode partitions: a length in tokens, 0 = the library's plan, "
                         "'balanced' = the batch's chunks spread evenly over the CUs; default "
                         "'auto': the library chooses from the batch's lengths "
                         "(pba_paged_decode_plan_ex with PBA_PARTITIONS_AUTO)")
    ap.add_argument("--decode", default="auto", choices=["auto", "plain", "shared"],
                    help="decode entry point: paged_decode, paged_decode_shared (shared-prefix "
                         "execution reuse), or auto = shared when the batch shares chunks")
    ap.add_argument("--shared-partition-tokens", type=int, default=1024,
                    help="piece length of the shared-prefix plan")
    ap.add_argument("--shared-tiles", type=int, default=2, choices=[1, 2, 4],
                    help="16-column tiles per chunk-first item of the shared-prefix plan")
    ap.add_argument("--shared-private", default="auto", choices=["auto", "pieces"],
                    help="private ranges of the shared-prefix plan: auto = four rows per "
                         "work-group when every range is short, pieces = a work-group per piece")
    ap.add_argument("--tables", default="dense", choices=["dense", "ragged"],
                    help="block tables as a dense [B, n_max] array or compact rows with offsets")
    ap.add_argument("--kernel-block", type=int, default=0,
                    help="decode through a kernel view of this many tokens per block (the "
                         "allocator blocks split; tables expanded by the library)")
    ap.add_argument("--kv", default="paged", choices=["paged", "contiguous", "contiguous-plain"],
                    help="K/V layout: the paged pool (block tables), a contiguous virtual "
                         "arena with pages mapped on demand (slot index, no block table), or "
                         "the same contiguous layout in one ordinary device allocation")
    ap.add_argument("--page-mib", type=float, default=2.0,
                    help="physical page size of the contiguous arena, MiB")
    ap.add_argument("--step", default="fused", choices=["fused", "separate"],
                    help="fused: the step's new tokens are appended by the decode call "
                         "(paged_decode_append) when each is its row's last position; "
                         "separate: kv_append, then the decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache decode timing (kernel traces of the warm launches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode call, which in a fused step still "
                         "appends the step's tokens (profiling runs)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as a HIP graph (measured slower than eager launches "
                         "for these steps on ROCm 7.2)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run block_copy over this many MiB "
                         "(a plain copy of known size for counter calibration)")
    return ap.parse_args()


def make_workload(name: str):
    import workloads as wl

    if name.startswith("lognormal_p"):
        return wl.lognormal(int(name[len("lognormal_p"):]))
    return getattr(wl, name)()


# ---------------------------------------------------------------------------
# The caller's side: run the script through the block manager.
# ---------------------------------------------------------------------------
@dataclass
class Plan:
    setup: List[Tuple]          # ("copy", src, dst) | ("append", slots, row_lo, row_hi)
    step_src: np.ndarray        # copy-on-write pairs of the step
    step_dst: np.ndarray
    step_slots: np.ndarray      # slots of the step's appended tokens
    step_rows: Tuple[int, int]  # their K/V rows in script order
    tables: np.ndarray          # int32 [B, max_blocks] of the decode batch
    seq_lens: np.ndarray        # int32 [B]
    n_writes: int


def plan_script(w) -> Plan:
    """Setup = every action before the script's trailing one-token appends;
    the step = those appends (with the copies they cause) and the decode."""
    import workloads as wl
    from block_table_attention_amd.blocks import BlockManager

    m = BlockManager(w.shape.num_blocks, w.shape.block_size, free_order=wl.fifo_order(w))
    n_tail = 0
    for act in reversed(w.actions):
        if act[0] != "append":
            break
        n_tail += 1
    first_step = len(w.actions) - n_tail
    setup: List[Tuple] = []
    src: List[int] = []
    dst: List[int] = []
    step_slots: List[np.ndarray] = []
    row = 0
    step_lo = None
    for i, act in enumerate(w.actions):
        kind = act[0]
        if kind == "new":
            m.new_request()
        elif kind == "fork":
            m.fork(act[1])
        elif kind == "release":
            m.release(act[1])
        else:
            n = act[2] if kind == "prefill" else 1
            slots, copies = m.append(act[1], n)
            if i >= first_step:
                step_lo = row if step_lo is None else step_lo
                src += [c[0] for c in copies]
                dst += [c[1] for c in copies]
                step_slots.append(slots)
            else:
                for s, d in copies:
                    setup.append(("copy", np.array([s], np.int32), np.array([d], np.int32)))
                setup.append(("append", slots, row, row + n))
            row += n
    step_lo = row if step_lo is None else step_lo
    return Plan(setup, np.array(src, np.int32), np.array(dst, np.int32),
                np.concatenate(step_slots) if step_slots else np.zeros(0, np.int64),
                (step_lo, row), m.block_tables(w.decode), m.seq_lens(w.decode), row)


def visible_slots(tables: np.ndarray, lens: np.ndarray, P: int) -> np.ndarray:
    """Physical slot of every (request, position < T) the decode reads."""
    out = []
    for r, T in enumerate(lens):
        t = np.arange(int(T), dtype=np.int64)
        out.append(tables[r, t // P].astype(np.int64) * P + t % P)
    return np.concatenate(out)


def step_rows_if_fusable(plan: Plan, P: int):
    """Decode row of each of the step's new tokens, in the step's order, when
    the decode call can append them (None otherwise): every new token is its
    row's last position (one token per row) in a block no other row of the
    batch reads -- the copy-on-write rule, so no work-group reads a position
    that another one writes."""
    if len(plan.step_slots) == 0:
        return None
    last = {int(plan.tables[r, (T - 1) // P]) * P + (T - 1) % P: r
            for r, T in enumerate(plan.seq_lens)}
    rows = [last.get(int(sl), -1) for sl in plan.step_slots]
    if min(rows) < 0 or len(set(rows)) != len(rows):
        return None
    refs = {}
    for r, T in enumerate(plan.seq_lens):
        for b in plan.tables[r, :-(-int(T) // P)]:
            refs[int(b)] = refs.get(int(b), 0) + 1
    if any(refs[int(sl) // P] != 1 for sl in plan.step_slots):
        return None
    return rows


def shared_step_rows(rows, order, host_plan, lens_sorted):
    """The same rows in the sharing order of a shared-prefix plan, or None
    when a new token lies outside its row's private range (a chunk's blocks
    are shared)."""
    pos = np.empty(len(order), dtype=np.int64)
    pos[order] = np.arange(len(order))
    rows = [int(pos[r]) for r in rows]
    if any(host_plan.row_private[r, 0] > lens_sorted[r] - 1 for r in rows):
        return None
    return rows


def decode_bytes(plan: Plan, shape):
    """(unique K/V bytes, logical K/V bytes, algorithmic bytes of one decode)."""
    P, Hq, Hkv, d = shape.block_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    es = 2 if shape.dtype == "bf16" else 4
    row = Hkv * d * 2 * es
    lens = plan.seq_lens
    B = len(lens)
    kv_unique = int(np.unique(visible_slots(plan.tables, lens, P)).size) * row
    kv_logical = int(lens.sum()) * row
    q = B * Hq * d * es
    out = B * Hq * d * 4 + B * Hq * 4
    tbl = int(sum(-(-int(T) // P) for T in lens)) * 4 + B * 4
    return kv_unique, kv_logical, kv_unique + q + out + tbl


def table_ledger(plan: Plan, P: int) -> dict:
    """Block-size accounting of the decode batch: tail slots (allocated but
    past T), and dense versus used block-table cells."""
    lens = plan.seq_lens.astype(np.int64)
    blocks = -(-lens // P)
    tail = int((blocks * P - lens).sum())
    return {"blocks_mapped": int(blocks.sum()), "tail_slots": tail,
            "tail_fraction": round(tail / float((blocks * P).sum()), 4),
            "table_cells_dense": int(len(lens) * plan.tables.shape[1]),
            "table_cells_used": int(blocks.sum())}


# The sources that decide a decode launch's HBM traffic: the kernels, the
# library's planner (partition plan, balanced or grid decomposition, workspace
# layout) and the caller-side helpers that choose the partitions and build the
# shared-prefix plan.
DIGEST_SOURCES = ("block_table_attention_amd/csrc/paged_decode.hip",
                  "block_table_attention_amd/csrc/pba_internal.h",
                  "block_table_attention_amd/csrc/pba_api.hip",
                  "block_table_attention_amd/csrc/plan.cpp",
                  "block_table_attention_amd/blocks.py")


def decode_source_digest(root: str = ROOT) -> str:
    """SHA-256 of the sources that decide the decode's traffic (DIGEST_SOURCES)
    with comments and whitespace removed: a profile stays valid across edits
    that change no code, and any code edit to the kernels or the planners
    voids it."""
    import hashlib
    import re

    parts = []
    for rel in DIGEST_SOURCES:
        path = os.path.join(root, rel)
        if not os.path.exists(path):
            parts.append(f"<missing {rel}>")
            continue
        text = open(path).read()
        if rel.endswith(".py"):
            text = re.sub(r"#[^\n]*", " ", text)
        else:
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
        parts.append(re.sub(r"\s+", " ", text).strip())
    return hashlib.sha256("\x00".join(parts).encode()).hexdigest()


def profiled_traffic(workload: str, root: str = ROOT):
    """HBM bytes per decode launch from the committed rocprofv3 summary, or None
    when there is none for this workload or the decode code or planners changed
    since."""
    import re

    path = os.path.join(root, "profiles", f"decode_bf16_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    m_h = re.search(r"decode_code_sha256: ([0-9a-f]{64})", text)
    if not (m_t and m_h) or m_h.group(1) != decode_source_digest(root):
        return None
    return int(m_t.group(1))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this implementation runs on one GPU; --gpus {args.gpus} is not "
              "supported (requests and kv heads shard without exchange, one long request "
              "would need an all-gather of partition states)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_table_attention_amd as pba

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration_mib:
        return copy_calibration(args, pba, torch, dev)
    names = WORKLOADS if args.sweep else [args.workload]
    for name in names:
        if args.kv.startswith("contiguous") and (name in BUNDLE_WORKLOADS or name == "tiny"):
            continue          # the contiguous arena path covers the bf16 single-layer workloads
        if name in BUNDLE_WORKLOADS:
            result = run_bundle(args, name, pba, torch, dev)
            if not (args.sweep or args.no_cpu_baseline):
                result["cpu_baseline"] = cpu_baseline_bundle(make_workload(name), args.cpu_seconds,
                                                             result["_kv_value_bytes"])
        elif args.kv.startswith("contiguous"):
            result = run_contiguous(args, name, pba, torch, dev)
            if not (args.sweep or args.no_cpu_baseline):
                w = make_workload(name)
                result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, result["_kv_value_bytes"])
        else:
            result = run_workload(args, name, pba, torch, dev)
            if not (args.sweep or args.no_cpu_baseline):
                w = make_workload(name)
                result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, result["_kv_value_bytes"])
        result.pop("_kv_value_bytes")
        print(json.dumps(result), flush=True)


def run_workload(args, name, pba, torch, dev):
    import workloads as wl

    w = make_workload(name)
    sh = w.shape
    P, Hq, Hkv, d = sh.block_size, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    tdtype = torch.bfloat16 if sh.dtype == "bf16" else torch.float32
    t0 = time.time()
    plan = plan_script(w)
    k_rows, v_rows = wl.kv_rows(w, plan.n_writes)
    print(f"[bench] {name}: planned the script and drew {plan.n_writes} K/V rows in "
          f"{time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def dev_bits(bits):
        view = np.int16 if sh.dtype == "bf16" else np.int32
        return torch.from_numpy(np.ascontiguousarray(bits).view(view)).view(tdtype).to(dev)

    k0, v0 = wl.pool_poison(w)
    pool = pba.KVPool(dev_bits(k0), dev_bits(v0))
    del k0, v0
    for op in plan.setup:
        if op[0] == "copy":
            pba.block_copy(pool, torch.from_numpy(op[1]).to(dev), torch.from_numpy(op[2]).to(dev))
        else:
            pba.kv_append(pool, torch.from_numpy(op[1]).to(dev), dev_bits(k_rows[op[2]:op[3]]),
                          dev_bits(v_rows[op[2]:op[3]]))
    lo, hi = plan.step_rows
    k_step, v_step = dev_bits(k_rows[lo:hi]), dev_bits(v_rows[lo:hi])
    del k_rows, v_rows
    step_slots = torch.from_numpy(plan.step_slots).to(dev)
    copy_src = torch.from_numpy(plan.step_src).to(dev)
    copy_dst = torch.from_numpy(plan.step_dst).to(dev)
    qb = wl.q_bits(w)
    B = len(plan.seq_lens)
    step_row = step_rows_if_fusable(plan, P)
    fusable = step_row is not None
    tables, lens_h = plan.tables, plan.seq_lens
    # Shared-prefix execution: the caller orders the batch so rows sharing
    # leading blocks are adjacent and describes the shared chunks.
    from block_table_attention_amd.blocks import shared_plan, sharing_order
    path = args.decode
    host_plan = None
    if path != "plain" and sh.dtype == "bf16":
        order = sharing_order(tables)
        cand = shared_plan(tables[order], lens_h[order], P, Hq // Hkv, args.shared_partition_tokens,
                           tiles_per_item=args.shared_tiles)
        if args.shared_private == "pieces":
            cand.private_tokens = 0
        if path == "shared" or any(b - a > 1 for a, b, _, _ in cand.chunks):
            tables, lens_h, qb, host_plan = tables[order], lens_h[order], qb[order], cand
            # Decode rows in sharing order; the fused step also needs each new
            # token inside its row's private range.
            if fusable:
                step_row = shared_step_rows(step_row, order, cand, lens_h)
                fusable = step_row is not None
    path = "shared" if host_plan is not None else "plain"
    q = dev_bits(qb)
    tab_d = torch.from_numpy(np.ascontiguousarray(tables)).to(dev)
    lens_d = torch.from_numpy(np.ascontiguousarray(lens_h)).to(dev)
    # Table encodings of the plain path: a kernel view of the pool (tables
    # expanded by the library) and/or compact rows with offsets.
    dpool = pool
    split = 0
    row_offsets = None
    table_cells = int(tab_d.numel())
    expand_us = None
    if host_plan is None and getattr(args, "kernel_block", 0):
        dpool = pool.kernel_view(args.kernel_block)
        split = dpool.split_log2
        tab_a = tab_d
        pba.expand_block_tables(tab_a, split)          # first launch loads the code
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tab_d = pba.expand_block_tables(tab_a, split)
        e1.record()
        torch.cuda.synchronize()
        expand_us = round(e0.elapsed_time(e1) * 1e3, 2)
    if host_plan is None and getattr(args, "tables", "dense") == "ragged":
        n_r = -(-lens_h.astype(np.int64) // P) << split   # whole expanded groups
        offs = np.zeros(len(n_r) + 1, dtype=np.int64)
        offs[1:] = np.cumsum(n_r)
        row_offsets = torch.from_numpy(offs).to(dev)
        tab_d = pba.pack_block_tables(tab_d, row_offsets, int(offs[-1]))
        table_cells = int(offs[-1])
    scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    mb = plan.tables.shape[1] << split
    # The bench is the caller: it knows the lengths and may pick the split.
    req_pt = args.partition_tokens
    # The library's dispatch decision for this batch, from a summary of its
    # lengths (PARTITIONS_AUTO), or for the partition length asked for.
    dispatch = pba.paged_decode_plan_ex(dpool, Hq, B, mb,
                                        pba.PARTITIONS_AUTO if req_pt == AUTO else req_pt,
                                        plan.seq_lens)
    req_pt = dispatch["partition_request"]
    if host_plan is None:
        pt, n_parts = pba.paged_decode_plan(dpool, Hq, B, mb, req_pt)
        # The balanced path reports no partition size, only its wave count.
        flat = req_pt == BALANCED and pt == 0
        ws_bytes = pba.paged_decode_workspace_bytes(dpool, Hq, B, mb, req_pt)
    else:
        flat = False
        splan = pba.SharedPlan.from_host(host_plan, dev)
        pt, n_parts = host_plan.partition_tokens, host_plan.max_slots
        ws_bytes = pba.paged_decode_shared_workspace_bytes(pool, Hq, B, mb, splan)
    # Zero-filled once: the library keeps the completion counters at zero.
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # --decode-only keeps the fused call: the profiled decode is the one the burst times.
    fused = args.step == "fused" and fusable and row_offsets is None
    if fused:
        ns = np.full(B, -1, dtype=np.int64)
        ns[step_row] = plan.step_slots
        new_slots = torch.from_numpy(ns).to(dev)
        knew = torch.zeros((B, Hkv, d), dtype=tdtype, device=dev)
        vnew = torch.zeros_like(knew)
        idx = torch.tensor(step_row, dtype=torch.int64, device=dev)
        knew[idx] = k_step
        vnew[idx] = v_step
    torch.cuda.synchronize()

    def decode(st=stream):
        if fused and host_plan is not None:   # (each call appends the same bytes again)
            pba.paged_decode_shared_append(pool, new_slots, knew, vnew, q, tab_d, lens_d, splan,
                                           scale, out=out, lse=lse, workspace=ws, stream=st)
        elif fused:
            pba.paged_decode_append(dpool, new_slots, knew, vnew, q, tab_d, lens_d, scale,
                                    out=out, lse=lse, partition_tokens=req_pt, workspace=ws,
                                    stream=st)
        elif host_plan is None and row_offsets is not None:
            pba.paged_decode_ragged(dpool, q, tab_d, row_offsets, lens_d, mb, scale, out=out,
                                    lse=lse, partition_tokens=req_pt, workspace=ws, stream=st)
        elif host_plan is None:
            pba.paged_decode(dpool, q, tab_d, lens_d, scale, out=out, lse=lse,
                             partition_tokens=req_pt, workspace=ws, stream=st)
        else:
            pba.paged_decode_shared(pool, q, tab_d, lens_d, splan, scale, out=out, lse=lse,
                                    workspace=ws, stream=st)

    def step(evs=None, st=stream):
        if evs is not None:
            evs[0].record(st)
        if not args.decode_only:
            pba.block_copy(pool, copy_src, copy_dst, stream=st)
            if evs is not None:
                evs[1].record(st)
            if not fused:
                pba.kv_append(pool, step_slots, k_step, v_step, stream=st)
        if evs is not None:
            evs[2].record(st)
        decode(st)
        if evs is not None:
            evs[3].record(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # The timed steps: K eager steps with no events inside, or with --graph one
    # HIP graph of the whole step (copy, append, decode) replayed K times.
    use_graph = args.graph and not args.decode_only
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(st=None)
        graph.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(K):
        if use_graph:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / K
    # Per-call breakdown: K eager steps with events between the calls (the
    # events add their own small gaps, so this pass is not the step time).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    if args.decode_only:
        copy_ms = append_ms = np.zeros(1)
    else:
        copy_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        append_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    # Roofline timing of the decode kernel: K launches back to back on the same
    # stream, HIP events only at the two ends (a per-launch event pair adds its
    # own idle gap to every launch).
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for _ in range(K):
        decode()
    b1.record(stream)
    torch.cuda.synchronize()
    dec_avg_ms = b0.elapsed_time(b1) / K
    warm1_ms, cold1_ms = (None, None) if args.no_cold else cold_launch_ms(torch, decode, stream, K)
    print(f"[bench] {name}: timed {K} steps ({'graph' if use_graph else 'eager'}): "
          f"{ms_per_step * 1e3:.1f} us/step, decode in eager step "
          f"{dec_ms.mean() * 1e3:.1f} us (p10 {np.percentile(dec_ms, 10) * 1e3:.1f}, "
          f"p90 {np.percentile(dec_ms, 90) * 1e3:.1f}); decode burst {dec_avg_ms * 1e3:.1f} us/launch",
          file=sys.stderr, flush=True)

    kv_unique, kv_logical, alg_bytes = decode_bytes(plan, sh)
    traffic = (profiled_traffic(name if host_plan is None else f"shared_{name}")
               if args.partition_tokens == AUTO and args.shared_partition_tokens == 1024
               and args.shared_tiles == 2 and args.shared_private == "auto"
               and args.tables == "dense" and args.kernel_block == 0 else None)
    step_kv_gbs = kv_unique / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (dec_avg_ms * 1e-3) / 1e9
    lens = plan.seq_lens
    es = 2 if sh.dtype == "bf16" else 4
    ctx = (f"context {int(lens[0])}" if lens.min() == lens.max()
           else f"context {int(lens.min())}..{int(lens.max())} (sum {int(lens.sum())})")
    result = {
        "metric": "paged decode: KV GB/s achieved (% of HBM peak) + query rows/s at 1 GPU",
        "value": round(step_kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sh.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q rounded to bf16; seeded free-FIFO block placement)",
        "config": {"workload": f"{name}: batch {B}, {ctx}, block_size {P}, {Hq} q-heads / "
                               f"{Hkv} kv-heads, head_dim {d}, {sh.dtype}, pool {sh.num_blocks} blocks",
                   "batch": B, "context_min": int(lens.min()), "context_max": int(lens.max()),
                   "context_sum": int(lens.sum()), "block_size": P, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": d, "pool_blocks": sh.num_blocks,
                   "partition_tokens": pt, "num_partitions": n_parts,
                   "partition_choice": "shared-prefix plan" if host_plan is not None else
                   ("library, from the lengths (PBA_PARTITIONS_AUTO)"
                    if args.partition_tokens == AUTO else "fixed by --partition-tokens"),
                   "dispatch": None if host_plan is not None else
                   {"decomposition": dispatch["decomposition"], "reason": dispatch["reason"],
                    "fallback": dispatch["fallback"],
                    "partition_request": dispatch["partition_request"]},
                   "decode_path": "balanced" if flat else path,
                   "tables": "ragged" if row_offsets is not None else "dense",
                   "table_cells": table_cells,
                   "kernel_block": P >> split,
                   "expand_us": expand_us,
                   "shared_plan": None if host_plan is None else
                   {"chunks": len(host_plan.chunks), "items": int(host_plan.items.shape[0]),
                    "max_slots": host_plan.max_slots,
                    "chunk_rows": int(sum(b - a for a, b, _, _ in host_plan.chunks)),
                    # Work items' 32-token chunk reads, and the partial states
                    # the launch writes (G x (d + 2) floats per row, slot and
                    # kv head), over all kv heads.
                    "chunk_visits": int(host_plan.chunk_visits) * Hkv,
                    "kv_rows_read": int(host_plan.kv_rows_read) * Hkv,
                    "partial_states": int(host_plan.partial_states) * Hkv,
                    "partial_state_bytes": int(host_plan.partial_states) * Hkv * (Hq // Hkv)
                    * (d + 2) * 4,
                    "private_tokens": host_plan.private_tokens,
                    "private_ranges": "four rows per work-group"
                    if 0 < host_plan.private_tokens <= 128 else "a work-group per piece"},
                   "step": f"block_copy({len(plan.step_src)} pairs) + " +
                           (f"{'paged_decode_shared_append' if host_plan is not None else 'paged_decode_append'}"
                            f"({len(plan.step_slots)} new tokens appended in the decode launch)"
                            if fused else
                            f"kv_append({len(plan.step_slots)} tokens) + "
                            f"{'paged_decode_shared' if host_plan is not None else 'paged_decode'}"),
                   "step_fused": fused,
                   "step_launch": "HIP graph replay" if use_graph else "eager"},
        "query_rows_per_s": round(B / (ms_per_step * 1e-3), 1),
        "hbm_peak_frac_step": round(step_kv_gbs / HBM_PEAK_GBS, 4),
        "decode_us": round(dec_avg_ms * 1e3, 2),
        "decode_us_cold": None if cold1_ms is None else round(cold1_ms * 1e3, 2),
        "cold_over_warm": None if cold1_ms is None else round(cold1_ms / warm1_ms, 3),
        "decode_us_in_step": round(float(dec_ms.mean()) * 1e3, 2),
        "decode_rows_per_s": round(B / (dec_avg_ms * 1e-3), 1),
        "decode_head_rows_per_s": round(B * Hq / (dec_avg_ms * 1e-3), 1),
        "append_us": None if fused else round(float(append_ms.mean()) * 1e3, 2),
        "copy_us": round(float(copy_ms.mean()) * 1e3, 2),
        # Bytes read + written by the step's append and copy, over their event-timed durations.
        "append_gbs": None if fused else
        round(len(plan.step_slots) * Hkv * d * es * 2 * 2 /
              max(float(append_ms.mean()) * 1e-3, 1e-12) / 1e9, 2),
        "copy_gbs": round(len(plan.step_src) * Hkv * P * d * es * 2 * 2 /
                          max(float(copy_ms.mean()) * 1e-3, 1e-12) / 1e9, 2),
        "kv_unique_bytes": kv_unique,
        "kv_logical_bytes": kv_logical,
        "kv_logical_gbs_decode": round(kv_logical / (dec_avg_ms * 1e-3) / 1e9, 2),
        "ledger": table_ledger(plan, P),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "frac_cold": None if cold1_ms is None else
                     round(alg_bytes / (cold1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel": (f"decode_bf16_shared_kernel<{d}> (chunk-first + sequence-first, "
                                "merge fused in" + (", the step's appends too)" if fused else ")"))
                     if host_plan is not None else
                               (f"decode_bf16_flat_kernel<{d}> (balanced chunk ranges, cut rows "
                                "merged in)" if flat else
                                f"decode_{sh.dtype}_kernel<{d}> (partition merge fused in"
                                + (", the step's appends too)" if fused else ")")),
                     "algorithmic_bytes_per_launch": alg_bytes},
        "_kv_value_bytes": kv_unique,
    }
    del pool, ws
    torch.cuda.empty_cache()
    return result


# ---------------------------------------------------------------------------
# Cache groups with a layer axis: the whole model's decode attention step.
# ---------------------------------------------------------------------------
@dataclass
class BundlePlan:
    setup: List[Tuple]          # ("copy", [(src, dst) per group]) | ("append", [slots per group], lo, hi)
    step_copies: List[Tuple[np.ndarray, np.ndarray]]   # per group
    step_slots: List[np.ndarray]                       # per group
    step_rows: Tuple[int, int]
    tables: List[np.ndarray]    # per group: int32 [B, max_blocks_g]
    seq_lens: np.ndarray
    n_writes: int


def plan_bundle_script(w) -> BundlePlan:
    """The BundleManager over the script; the step is its trailing appends."""
    import workloads as wl
    from block_table_attention_amd.blocks import BundleManager

    G = len(w.groups)
    m = BundleManager([g.num_blocks for g in w.groups], [g.block_size for g in w.groups],
                      free_orders=wl.bundle_fifo_orders(w))
    n_tail = 0
    for act in reversed(w.actions):
        if act[0] != "append":
            break
        n_tail += 1
    first_step = len(w.actions) - n_tail
    setup: List[Tuple] = []
    step_src = [[] for _ in range(G)]
    step_dst = [[] for _ in range(G)]
    step_slots = [[] for _ in range(G)]
    row = 0
    step_lo = None
    for i, act in enumerate(w.actions):
        kind = act[0]
        if kind == "new":
            m.new_request()
        elif kind == "fork":
            m.fork(act[1])
        elif kind == "release":
            m.release(act[1])
        else:
            n = act[2] if kind == "prefill" else 1
            slots, copies = m.append(act[1], n)
            if i >= first_step:
                step_lo = row if step_lo is None else step_lo
                for g in range(G):
                    step_src[g] += [c[0] for c in copies[g]]
                    step_dst[g] += [c[1] for c in copies[g]]
                    step_slots[g].append(slots[g])
            else:
                if any(copies):
                    setup.append(("copy", [(np.array([c[0] for c in copies[g]], np.int32),
                                            np.array([c[1] for c in copies[g]], np.int32))
                                           for g in range(G)]))
                setup.append(("append", slots, row, row + n))
            row += n
    step_lo = row if step_lo is None else step_lo
    return BundlePlan(setup,
                      [(np.array(step_src[g], np.int32), np.array(step_dst[g], np.int32))
                       for g in range(G)],
                      [np.concatenate(step_slots[g]) if step_slots[g] else np.zeros(0, np.int64)
                       for g in range(G)],
                      (step_lo, row), m.block_tables(w.decode), m.seq_lens(w.decode), row)


def run_bundle(args, name, pba, torch, dev):
    """One decode step of every layer: block_copy_bundle of the step's
    copy-on-write bundles, kv_append_bundle of the step's tokens into every
    layer of every group, then paged_decode of each layer through its group's
    layer pool and block table."""
    import workloads as wl

    w = make_workload(name)
    G = len(w.groups)
    Hq, Hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    t0 = time.time()
    plan = plan_bundle_script(w)
    rows = [wl.bundle_rows(w, g) for g in range(G)]
    print(f"[bench] {name}: planned the script and drew {plan.n_writes} rows x "
          f"{w.total_layers} layers in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def dev_bits(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    groups = []
    for g, gs in enumerate(w.groups):
        k0, v0 = wl.bundle_poison(w, g)
        lead = (gs.layers, gs.num_blocks) if gs.layer_major else (gs.num_blocks, gs.layers)
        k = dev_bits(k0).view(lead + (Hkv, gs.block_size, d))
        v = dev_bits(v0).view(lead + (Hkv, d, gs.block_size))
        groups.append(pba.KVGroup(k, v, gs.layer_major))
        del k0, v0
    rows_dev = [(dev_bits(k), dev_bits(v)) for k, v in rows]
    del rows
    for op in plan.setup:
        if op[0] == "copy":
            pba.block_copy_bundle(groups, [torch.from_numpy(s).to(dev) for s, _ in op[1]],
                                  [torch.from_numpy(t).to(dev) for _, t in op[1]])
        else:
            pba.kv_append_bundle(groups, [torch.from_numpy(s).to(dev) for s in op[1]],
                                 [r[0][op[2]:op[3]] for r in rows_dev],
                                 [r[1][op[2]:op[3]] for r in rows_dev])
    lo, hi = plan.step_rows
    k_step = [r[0][lo:hi].contiguous() for r in rows_dev]
    v_step = [r[1][lo:hi].contiguous() for r in rows_dev]
    k_step_l = [[k[:, l].contiguous() for l in range(k.shape[1])] for k in k_step]
    v_step_l = [[v[:, l].contiguous() for l in range(v.shape[1])] for v in v_step]
    del rows_dev
    slots = [torch.from_numpy(s).to(dev) for s in plan.step_slots]
    csrc = [torch.from_numpy(s).to(dev) for s, _ in plan.step_copies]
    cdst = [torch.from_numpy(t).to(dev) for _, t in plan.step_copies]
    q_all = dev_bits(wl.bundle_q_bits(w))           # [layers, B, Hq, d]
    B = len(plan.seq_lens)
    lens_d = torch.from_numpy(plan.seq_lens).to(dev)
    tabs = [torch.from_numpy(t).to(dev) for t in plan.tables]
    layer_pools = [(g, grp.layer(l)) for g, grp in enumerate(groups) for l in range(grp.num_layers)]
    scale = 1.0 / math.sqrt(d)
    req_pt = args.partition_tokens
    mbs = [t.shape[1] for t in plan.tables]
    if req_pt == AUTO:
        req_pt = pba.paged_decode_plan_ex(layer_pools[0][1], Hq, B, mbs[0], pba.PARTITIONS_AUTO,
                                          plan.seq_lens)["partition_request"]
    ws_bytes = max(pba.paged_decode_workspace_bytes(lp, Hq, B, mbs[g], req_pt) for g, lp in layer_pools)
    pt, n_parts = pba.paged_decode_plan(layer_pools[0][1], Hq, B, mbs[0], req_pt)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty((w.total_layers, B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.total_layers, B, Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def decode_layer(i, st=stream):
        g, lp = layer_pools[i]
        pba.paged_decode(lp, q_all[i], tabs[g], lens_d, scale, out=out[i], lse=lse[i],
                         partition_tokens=req_pt, workspace=ws, stream=st)

    def copies(st=stream):
        pba.block_copy_bundle(groups, csrc, cdst, stream=st)

    def appends(st=stream):
        pba.kv_append_bundle(groups, slots, k_step, v_step, stream=st)

    def copies_per_layer(st=stream):
        for g, grp in enumerate(groups):
            if csrc[g].numel():
                for l in range(grp.num_layers):
                    pba.block_copy(grp.layer(l), csrc[g], cdst[g], stream=st)

    def appends_per_layer(st=stream):
        for g, grp in enumerate(groups):
            for l in range(grp.num_layers):
                pba.kv_append(layer_pools_by_group[g][l], slots[g], k_step_l[g][l], v_step_l[g][l],
                              stream=st)

    layer_pools_by_group = [[grp.layer(l) for l in range(grp.num_layers)] for grp in groups]

    def step(evs=None, st=stream):
        if evs is not None:
            evs[0].record(st)
        copies(st)
        if evs is not None:
            evs[1].record(st)
        appends(st)
        if evs is not None:
            evs[2].record(st)
        for i in range(len(layer_pools)):
            decode_layer(i, st)
        if evs is not None:
            evs[3].record(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t_start = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / K
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    copy_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    append_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    dec_all_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])

    def burst(fn, reps):
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        b0.record(stream)
        for _ in range(reps):
            fn()
        b1.record(stream)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) / reps

    # The burst cycles through all layers, so each layer's rows have left the
    # caches (the other layers' rows pass through them) when it is decoded again.
    L = len(layer_pools)
    dec_avg_ms = burst(lambda: [decode_layer(i) for i in range(L)], K) / L
    copy_fused = burst(copies, K)
    copy_split = burst(copies_per_layer, K)
    app_fused = burst(appends, K)
    app_split = burst(appends_per_layer, K)
    print(f"[bench] {name}: {ms_per_step * 1e3:.1f} us/step; decode {dec_avg_ms * 1e3:.1f} us/layer; "
          f"copy {copy_fused * 1e3:.1f} us fused vs {copy_split * 1e3:.1f} per layer; append "
          f"{app_fused * 1e3:.1f} us fused vs {app_split * 1e3:.1f} per layer",
          file=sys.stderr, flush=True)

    # Bytes: one layer's decode reads every unique visible row of its group.
    lens = plan.seq_lens
    P = w.groups[0].block_size
    row_layer = Hkv * d * 2 * 2
    uniq = [int(np.unique(visible_slots(plan.tables[g], lens, w.groups[g].block_size)).size)
            for g in range(G)]
    kv_unique = sum(uniq[g] * row_layer * w.groups[g].layers for g in range(G))
    kv_logical = int(lens.sum()) * row_layer * w.total_layers
    small = B * Hq * d * 2 + B * Hq * d * 4 + B * Hq * 4 + B * 4
    alg_layer = [uniq[g] * row_layer + small + int(sum(-(-int(T) // w.groups[g].block_size)
                                                      for T in lens)) * 4 for g in range(G)]
    alg_avg = sum(alg_layer[g] * w.groups[g].layers for g in range(G)) / w.total_layers
    achieved = alg_avg / (dec_avg_ms * 1e-3) / 1e9
    traffic = profiled_traffic(name) if args.partition_tokens == AUTO else None
    step_kv_gbs = kv_unique / (ms_per_step * 1e-3) / 1e9
    n_copy = [int(s.numel()) for s in csrc]
    bundle_bytes = sum(gs.layers * Hkv * gs.block_size * d * 2 * 2 for gs in w.groups)
    result = {
        "metric": "paged decode: KV GB/s achieved (% of HBM peak) + query rows/s at 1 GPU",
        "value": round(step_kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q rounded to bf16; seeded free-FIFO block placement)",
        "config": {"workload": f"{name}: {w.total_layers} layers in {G} cache groups "
                               f"({', '.join(f'{gs.layers} layers P={gs.block_size} ' + ('layer' if gs.layer_major else 'block') + '-major' for gs in w.groups)}), "
                               f"batch {B}, context {int(lens.min())}..{int(lens.max())} "
                               f"(sum {int(lens.sum())}), {Hq} q-heads / {Hkv} kv-heads, head_dim {d}, "
                               f"bf16, {w.groups[0].num_blocks} blocks per group",
                   "batch": B, "layers": w.total_layers, "groups": G,
                   "context_min": int(lens.min()), "context_max": int(lens.max()),
                   "context_sum": int(lens.sum()), "block_size": P, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": d, "partition_tokens": pt,
                   "num_partitions": n_parts, "bundle_bytes": bundle_bytes,
                   "step": f"block_copy_bundle({n_copy} pairs per group) + kv_append_bundle("
                           f"{int(slots[0].numel())} tokens x {w.total_layers} layers) + "
                           f"{w.total_layers} x paged_decode",
                   "step_launch": "eager"},
        "query_rows_per_s": round(B / (ms_per_step * 1e-3), 1),
        "hbm_peak_frac_step": round(step_kv_gbs / HBM_PEAK_GBS, 4),
        "decode_us": round(dec_avg_ms * 1e3, 2),
        "decode_all_layers_us_in_step": round(float(dec_all_ms.mean()) * 1e3, 2),
        "append_us": round(float(append_ms.mean()) * 1e3, 2),
        "copy_us": round(float(copy_ms.mean()) * 1e3, 2),
        "copy_bundle_us": round(copy_fused * 1e3, 2),
        "copy_per_layer_calls_us": round(copy_split * 1e3, 2),
        "append_bundle_us": round(app_fused * 1e3, 2),
        "append_per_layer_calls_us": round(app_split * 1e3, 2),
        "kv_unique_bytes": kv_unique,
        "kv_logical_bytes": kv_logical,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": f"decode_bf16_kernel<{d}> (one launch per layer, merge fused in)",
                     "algorithmic_bytes_per_launch": int(round(alg_avg))},
        "_kv_value_bytes": kv_unique,
    }
    del groups, ws
    torch.cuda.empty_cache()
    return result


def run_contiguous(args, name, pba, torch, dev):
    """The same decode batch over a contiguous virtual arena (vAttention
    layout): one slot per request, pages mapped for each request's rows, no
    block table.  A step is kv_append of the step's tokens (slot ids in the
    arena) + paged_decode_contiguous.  The arena's rows are synthetic draws
    written once (the decode's time does not depend on their values); requests
    that share blocks in the paged pool each hold their own rows here."""
    w = make_workload(name)
    sh = w.shape
    if sh.dtype != "bf16":
        raise SystemExit(f"{name}: the contiguous decode is bf16 only")
    Hq, Hkv, d = sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    plan = plan_script(w)
    lens = plan.seq_lens.astype(np.int64)
    B = len(lens)
    P = 64 if sh.block_size >= 64 else sh.block_size
    page = int(args.page_mib * (1 << 20))
    virtual = args.kv == "contiguous"
    if virtual:
        arena = pba.VKVArena(1, B, int(lens.max()), Hkv, d, P, page, dtype=torch.bfloat16,
                             device=dev)
        t0 = time.perf_counter()
        for r in range(B):
            arena.map(r, int(lens[r]))
        map_s = time.perf_counter() - t0
        led = arena.ledgers()
        bundles = led["bundle_maps"]
        pool = arena.layer(0)
        bps = arena.blocks_per_slot
        slot_ids = arena.slot_ids
    else:                     # the same layout in one device allocation, no VMM
        bps = int(-(-int(lens.max()) // P))
        pool = pba.KVPool.empty(B * bps, P, Hkv, d, torch.bfloat16, dev)
        slot_ids = lambda r, t: r * bps * P + t
        map_s, bundles, led = 0.0, 0, None
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    for r in range(B):            # rows 0 .. T-2; the step appends row T-1
        n = int(lens[r]) - 1
        if n <= 0:
            continue
        ids = torch.from_numpy(slot_ids(r, np.arange(n, dtype=np.int64))).to(dev)
        k = torch.randn((n, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((n, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        pba.kv_append(pool, ids, k, v)
    step_ids = torch.from_numpy(slot_ids(np.arange(B, dtype=np.int64), lens - 1)).to(dev)
    k_step = torch.randn((B, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    v_step = torch.randn((B, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    slot_index = torch.arange(B, dtype=torch.int32, device=dev)
    lens_d = torch.from_numpy(lens.astype(np.int32)).to(dev)
    req_pt = args.partition_tokens
    if req_pt == AUTO:
        req_pt = pba.paged_decode_plan_ex(pool, Hq, B, bps, pba.PARTITIONS_AUTO,
                                          lens)["partition_request"]
    pt, n_parts = pba.paged_decode_plan(pool, Hq, B, bps, req_pt)
    ws = torch.zeros(max(pba.paged_decode_workspace_bytes(pool, Hq, B, bps, req_pt), 16),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream()

    def decode():
        pba.paged_decode_contiguous(pool, q, slot_index, bps, lens_d, scale, out=out, lse=lse,
                                    partition_tokens=req_pt, workspace=ws)

    def step():
        pba.kv_append(pool, step_ids, k_step, v_step)
        decode()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t_start = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / K
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for _ in range(K):
        decode()
    b1.record(stream)
    torch.cuda.synchronize()
    dec_avg_ms = b0.elapsed_time(b1) / K
    warm1_ms, cold1_ms = (None, None) if args.no_cold else cold_launch_ms(torch, decode, stream, K)
    row = Hkv * d * 2 * 2
    kv_bytes = int(lens.sum()) * row
    alg = kv_bytes + B * Hq * d * 2 + B * Hq * d * 4 + B * Hq * 4 + B * 4 * 2
    achieved = alg / (dec_avg_ms * 1e-3) / 1e9
    step_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    print(f"[bench] {name} {args.kv}: {ms_per_step * 1e3:.1f} us/step, decode burst "
          f"{dec_avg_ms * 1e3:.1f} us/launch; mapped {bundles} page bundles in "
          f"{map_s * 1e3:.1f} ms", file=sys.stderr, flush=True)
    traffic = profiled_traffic(f"contig_{name}") if virtual and args.partition_tokens == AUTO and \
        args.page_mib == 2.0 else None
    result = {
        "metric": "paged decode: KV GB/s achieved (% of HBM peak) + query rows/s at 1 GPU",
        "value": round(step_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) K/V/q rounded to bf16, drawn on the device)",
        "config": {"workload": f"{name} over a contiguous "
                               f"{'virtual arena' if virtual else 'device buffer'}: batch {B}, context "
                               f"{int(lens.min())}..{int(lens.max())} (sum {int(lens.sum())}), "
                               f"tile {P} rows, {Hq} q-heads / {Hkv} kv-heads, head_dim {d}, "
                               f"pages of {page >> 10} KiB",
                   "kv_layout": args.kv, "batch": B, "context_sum": int(lens.sum()),
                   "tile_rows": P, "blocks_per_slot": bps, "page_bytes": page,
                   "partition_tokens": pt, "num_partitions": n_parts,
                   "decode_path": "balanced" if req_pt == BALANCED and pt == 0 else "plain",
                   "step": f"kv_append({B} tokens) + paged_decode_contiguous",
                   "step_launch": "eager"},
        "query_rows_per_s": round(B / (ms_per_step * 1e-3), 1),
        "decode_us": round(dec_avg_ms * 1e3, 2),
        "decode_us_cold": None if cold1_ms is None else round(cold1_ms * 1e3, 2),
        "cold_over_warm": None if cold1_ms is None else round(cold1_ms / warm1_ms, 3),
        "arena": None if not virtual else
                 {"reserved_bytes": led["reserved_bytes"], "mapped_bytes": led["mapped_bytes"],
                  "pool_bytes": led["pool_bytes"], "page_bundles_mapped": bundles,
                  "map_ms_total": round(map_s * 1e3, 2),
                  "map_us_per_bundle": round(map_s * 1e6 / max(bundles, 1), 1),
                  "mapped_over_rows": round(led["mapped_bytes"] / kv_bytes, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "frac_cold": None if cold1_ms is None else
                     round(alg / (cold1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel": (f"decode_bf16_flat_kernel<{d}, contiguous> (slot index, balanced "
                                "chunk ranges)" if req_pt == BALANCED and pt == 0 else
                                f"decode_bf16_kernel<{d}, contiguous> (slot index, no block table)"),
                     "algorithmic_bytes_per_launch": alg},
        "_kv_value_bytes": kv_bytes,
    }
    del pool
    if virtual:
        arena.close()
    torch.cuda.empty_cache()
    return result


def host_cpu():
    """(usable cores, CPU model name) of this host: the cores from the
    process's affinity mask, the model from lscpu (else /proc/cpuinfo)."""
    import subprocess

    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        out = subprocess.run(["lscpu"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                             text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.split(":")[0].strip() == "Model name":
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    return cores, model or "unknown"


def timed_oracle_rows(run_row, n_rows, seconds, threads):
    """Whole decode rows of the oracle, in batch order, until about `seconds`
    have elapsed, with `threads` BLAS threads: (rows done, elapsed s)."""
    from threadpoolctl import threadpool_limits

    done = 0
    with threadpool_limits(limits=threads):
        start = time.perf_counter()
        r = 0
        while True:
            run_row(r)
            done += 1
            r = (r + 1) % n_rows
            if time.perf_counter() - start >= seconds:
                break
        el = time.perf_counter() - start
    return done, el


def cpu_baseline_bundle(w, seconds, kv_bytes_total):
    """The CPU oracle on a bounded sample: whole decode rows of layer 0 (a
    single-layer oracle pool of the first group, replayed with that layer's
    rows), scaled to the bytes of every layer."""

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import execute_bundle
    import workloads as wl
    from oracle import attention as att
    from oracle.pool import BitPool

    t0 = time.time()
    ex = execute_bundle(w)
    gs = w.groups[0]
    k_rows, v_rows = wl.bundle_rows(w, 0)
    H, d, P = w.num_kv_heads, w.head_dim, gs.block_size
    pool = BitPool(np.zeros((gs.num_blocks, H, P, d), np.uint16),
                   np.zeros((gs.num_blocks, H, d, P), np.uint16), w.dtype)
    for op in ex.ops:
        if op[0] == "append":
            pool.kv_append(op[1][0], k_rows[op[2]:op[3], 0], v_rows[op[2]:op[3], 0])
        elif op[1][0][0].size:
            pool.block_copy(op[1][0][0], op[1][0][1])
    del k_rows, v_rows
    qb = wl.bundle_q_bits(w)[0]
    scale = 1.0 / math.sqrt(d)
    print(f"[bench] cpu oracle set-up {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    B = len(w.decode)
    tables0 = list(ex.tables[0])

    def run_row(r):
        att.paged_decode(pool, qb, tables0, ex.seq_lens, scale, rows=[(r, h) for h in range(H)])

    cores, model = host_cpu()
    done, el = timed_oracle_rows(run_row, B, seconds, cores)
    done1, el1 = timed_oracle_rows(run_row, B, seconds / 2, 1)
    per_layer = kv_bytes_total / w.total_layers
    return {"value": round(per_layer * done / B / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "cpu_model": model, "rows_per_s": round(done / el, 3),
            "value_1_thread": round(per_layer * done1 / B / el1 / 1e9, 4),
            "rows_per_s_1_thread": round(done1 / el1, 3),
            "sample": f"{done} whole decode rows of layer 0 (all {w.num_q_heads} q-heads) of the "
                      f"same workload, binary64 numpy oracle, {cores} BLAS threads (the host's "
                      f"usable cores), {el:.1f}s; then {done1} rows with 1 BLAS thread in "
                      f"{el1:.1f}s; bytes per row scaled to one layer"}


def cpu_baseline(w, seconds, kv_bytes_total):
    """Time the CPU oracle (binary64 numpy) on a bounded sample of the same
    workload: whole decode rows (all kv heads), in batch order, until about
    `seconds` have elapsed.  Bytes are the same count as the GPU value, scaled by
    the fraction of the batch done."""

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import execute, oracle_pool
    import workloads as wl
    from oracle import attention as att

    t0 = time.time()
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    del k_rows, v_rows
    qb = wl.q_bits(w)
    scale = 1.0 / math.sqrt(w.shape.head_dim)
    print(f"[bench] cpu oracle set-up {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    Hkv = w.shape.num_kv_heads
    B = len(w.decode)
    tables = list(ex.tables)

    def run_row(r):
        att.paged_decode(opool, qb, tables, ex.seq_lens, scale, rows=[(r, h) for h in range(Hkv)])

    cores, model = host_cpu()
    done_rows, el = timed_oracle_rows(run_row, B, seconds, cores)
    done1, el1 = timed_oracle_rows(run_row, B, seconds / 2, 1)
    lens = ex.seq_lens
    return {"value": round(kv_bytes_total * done_rows / B / el / 1e9, 4), "unit": "GB/s",
            "cores": cores, "kind": "oracle", "cpu_model": model,
            "rows_per_s": round(done_rows / el, 3),
            "value_1_thread": round(kv_bytes_total * done1 / B / el1 / 1e9, 4),
            "rows_per_s_1_thread": round(done1 / el1, 3),
            "sample": f"{done_rows} whole decode rows (all {w.shape.num_q_heads} q-heads; contexts "
                      f"{int(lens.min())}..{int(lens.max())}) of the same workload, binary64 numpy "
                      f"oracle, {cores} BLAS threads (the host's usable cores), {el:.1f}s; then "
                      f"{done1} rows with 1 BLAS thread in {el1:.1f}s"}


def copy_calibration(args, pba, torch, dev):
    """A plain copy of known size: block_copy over N MiB of whole blocks."""
    P, H, d = 64, 8, 128
    block_bytes = 2 * H * P * d * 2
    n = max(1, args.copy_calibration_mib * (1 << 20) // block_bytes)
    pool = pba.KVPool.empty(2 * n, P, H, d, torch.bfloat16, dev)
    src = torch.arange(0, n, dtype=torch.int32, device=dev)
    dst = torch.arange(n, 2 * n, dtype=torch.int32, device=dev)
    for _ in range(3):
        pba.block_copy(pool, src, dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    reps = 10
    for _ in range(reps):
        pba.block_copy(pool, src, dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_calibration": {"bytes_read": n * block_bytes, "bytes_written": n * block_bytes,
                                           "us": round(ms * 1e3, 2),
                                           "GBps_rw": round(2 * n * block_bytes / (ms * 1e-3) / 1e9, 1)}}))


if __name__ == "__main__":
    main()
