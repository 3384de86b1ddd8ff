#!/usr/bin/env python3
"""Benchmark: one decode step of paged attention on one MI355X.

A step is one pass of the whole hot path over the batch: kv_append of one new
token per request, block_copy of the step's copy-on-write pairs (none in the
long-context workloads), and paged_decode of one query row per request.

Default workload: long16k -- 8 requests x 16,384 tokens of context at decode
(16,383 prefilled + 1 appended per step), block size 64, 64 q-heads / 8
kv-heads (GQA 8), head_dim 128, bf16 K/V, pool of 4096 blocks (1 GiB).  All
inputs are seeded synthetic data and resident in HBM before timing starts.

Prints one JSON line: metric, value (K/V GB/s of a whole step), step time,
query rows/s, the roofline of the decode kernel (its average launch time over
a back-to-back burst, timed with HIP events on its stream, against HBM peak),
and cpu_baseline (the CPU oracle timed on a bounded sample of the same
workload).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long16k", choices=["long16k", "long64k", "batch32"])
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode call (profiling runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run block_copy over this many MiB "
                         "(a plain copy of known size for counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# The caller's side of allocation for workloads without sharing: a fresh pool
# hands out blocks from its free FIFO head, request by request.
# ---------------------------------------------------------------------------
def fresh_pool_layout(order: np.ndarray, lengths, P: int):
    """Block tables [B, max_blocks] (int32) for a fresh pool, request-major."""
    need = [-(-int(T) // P) for T in lengths]
    tables = np.full((len(lengths), max(need)), -1, dtype=np.int32)
    cursor = 0
    for r, n in enumerate(need):
        tables[r, :n] = order[cursor:cursor + n]
        cursor += n
    return tables


def slots_for(tables: np.ndarray, r: int, positions: np.ndarray, P: int) -> np.ndarray:
    return tables[r, positions // P].astype(np.int64) * P + positions % P


def decode_bytes(lengths, P, Hq, Hkv, d, esize):
    kv = int(sum(lengths)) * Hkv * d * 2 * esize
    q = len(lengths) * Hq * d * esize
    out = len(lengths) * Hq * d * 4 + len(lengths) * Hq * 4
    tbl = sum(-(-int(T) // P) for T in lengths) * 4 + len(lengths) * 4
    return kv, kv + q + out + tbl


def profiled_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 summary, or None
    when there is none for this workload or the decode source changed since."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"decode_bf16_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    m_h = re.search(r"decode_source_sha256: ([0-9a-f]{64})", text)
    if not (m_t and m_h):
        return None
    csrc = os.path.join(ROOT, "block_table_attention_amd", "csrc")
    blob = b"".join(open(os.path.join(csrc, f), "rb").read()
                    for f in ("paged_decode.hip", "pba_internal.h"))
    if hashlib.sha256(blob).hexdigest() != m_h.group(1):
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
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration_mib:
        return copy_calibration(args, pba, torch, dev)

    w = {"long16k": wl.long16k, "long64k": wl.long64k, "batch32": wl.batch32}[args.workload]()
    sh = w.shape
    P, Hq, Hkv, d = sh.block_size, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    tdtype = torch.bfloat16 if sh.dtype == "bf16" else torch.float32
    esize = 2 if sh.dtype == "bf16" else 4

    # Script shape of these workloads: per request a prefill, then one
    # appended token per request (the step's append).
    prefill = [a[2] for a in w.actions if a[0] == "prefill"]
    B = len(prefill)
    ctx = [T + 1 for T in prefill]          # context at decode
    order = wl.fifo_order(w)
    tables = fresh_pool_layout(order, ctx, P)
    n_pre = sum(prefill)
    t0 = time.time()
    k_rows, v_rows = wl.kv_rows(w, n_pre + B)
    print(f"[bench] drew {n_pre + B} K/V rows in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def dev_bits(bits):
        view = np.int16 if sh.dtype == "bf16" else np.int32
        return torch.from_numpy(np.ascontiguousarray(bits).view(view)).view(tdtype).to(dev)

    k0, v0 = wl.pool_poison(w)
    pool = pba.KVPool(dev_bits(k0), dev_bits(v0))
    del k0, v0
    pre_slots = np.concatenate([slots_for(tables, r, np.arange(prefill[r]), P) for r in range(B)])
    step_slots = np.array([slots_for(tables, r, np.array([prefill[r]]), P)[0] for r in range(B)])
    pba.kv_append(pool, torch.from_numpy(pre_slots).to(dev), dev_bits(k_rows[:n_pre]),
                  dev_bits(v_rows[:n_pre]))
    k_step, v_step = dev_bits(k_rows[n_pre:]), dev_bits(v_rows[n_pre:])
    step_slots_d = torch.from_numpy(step_slots).to(dev)
    copy_src = torch.empty(0, dtype=torch.int32, device=dev)
    copy_dst = torch.empty(0, dtype=torch.int32, device=dev)
    qb = wl.q_bits(w)
    q = dev_bits(qb)
    tab_d = torch.from_numpy(tables).to(dev)
    lens_d = torch.from_numpy(np.array(ctx, dtype=np.int32)).to(dev)
    scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    pt, n_parts = pba.paged_decode_plan(pool, Hq, B, tables.shape[1], args.partition_tokens)
    ws_bytes = pba.paged_decode_workspace_bytes(pool, Hq, B, tables.shape[1], args.partition_tokens)
    # Zero-filled once: the library keeps the completion counters at zero.
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev0=None, ev1=None):
        if not args.decode_only:
            pba.kv_append(pool, step_slots_d, k_step, v_step, stream=stream)
            pba.block_copy(pool, copy_src, copy_dst, stream=stream)
        if ev0 is not None:
            ev0.record(stream)
        pba.paged_decode(pool, q, tab_d, lens_d, scale, out=out, lse=lse,
                         partition_tokens=args.partition_tokens, workspace=ws, stream=stream)
        if ev1 is not None:
            ev1.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(*evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = elapsed * 1e3 / K
    dec_step_ms = float(np.mean(dec_ms))
    # Roofline timing of the decode kernel: K launches back to back on the same
    # stream, HIP events only at the two ends (a per-launch event pair adds its
    # own idle gap to every launch).
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for _ in range(K):
        pba.paged_decode(pool, q, tab_d, lens_d, scale, out=out, lse=lse,
                         partition_tokens=args.partition_tokens, workspace=ws, stream=stream)
    b1.record(stream)
    torch.cuda.synchronize()
    dec_avg_ms = b0.elapsed_time(b1) / K
    print(f"[bench] timed {K} steps: {ms_per_step * 1e3:.1f} us/step, decode in step "
          f"{dec_step_ms * 1e3:.1f} us (p10 {np.percentile(dec_ms, 10) * 1e3:.1f}, "
          f"p90 {np.percentile(dec_ms, 90) * 1e3:.1f}); decode burst {dec_avg_ms * 1e3:.1f} us/launch",
          file=sys.stderr, flush=True)

    kv_bytes, alg_bytes = decode_bytes(ctx, P, Hq, Hkv, d, esize)
    traffic = profiled_traffic(w.name) if args.partition_tokens == 0 else None
    step_kv_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (dec_avg_ms * 1e-3) / 1e9
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
        "config": {"workload": f"{w.name}: batch {B} x context {ctx[0]}, block_size {P}, "
                               f"{Hq} q-heads / {Hkv} kv-heads, head_dim {d}, {sh.dtype}, "
                               f"pool {sh.num_blocks} blocks",
                   "batch": B, "context": ctx[0], "block_size": P, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": d, "pool_blocks": sh.num_blocks,
                   "partition_tokens": pt, "num_partitions": n_parts,
                   "step": "kv_append(1 token/request) + block_copy(0 pairs) + paged_decode"},
        "query_rows_per_s": round(B / (ms_per_step * 1e-3), 1),
        "hbm_peak_frac_step": round(step_kv_gbs / HBM_PEAK_GBS, 4),
        "decode_us": round(dec_avg_ms * 1e3, 2),
        "decode_us_in_step": round(dec_step_ms * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode_bf16_kernel<128> (partition merge fused in)",
                     "algorithmic_bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, ctx, args.cpu_seconds, kv_bytes, B)
    print(json.dumps(result), flush=True)


def cpu_baseline(w, ctx, seconds, kv_bytes_total, B):
    """Time the CPU oracle (binary64 numpy) on a bounded sample of the same
    workload: whole requests, all kv heads, until ~`seconds` have elapsed."""
    from threadpoolctl import threadpool_limits

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
    done_rows = 0
    done_bytes = 0
    with threadpool_limits(limits=1):
        start = time.perf_counter()
        r = 0
        while True:
            att.paged_decode(opool, qb, list(ex.tables), ex.seq_lens, scale,
                             rows=[(r, h) for h in range(Hkv)])
            done_rows += 1
            done_bytes += kv_bytes_total // B
            r = (r + 1) % B
            if time.perf_counter() - start >= seconds:
                break
        el = time.perf_counter() - start
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "rows_per_s": round(done_rows / el, 3),
            "sample": f"{done_rows} whole decode rows (all {w.shape.num_q_heads} q-heads, context "
                      f"{ctx[0]}) of the same workload, binary64 numpy oracle, 1 BLAS thread, "
                      f"{el:.1f}s"}


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
