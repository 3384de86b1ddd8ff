"""GPU test of the allocation-free decode entry point (pba_paged_decode_noalloc)
through the C ABI: its output against pba_paged_decode's with a caller
workspace -- bitwise equal (same kernels, same plan) and within 2e-3 of the
binary64 oracle -- on calls in a row over different layouts, the later ones
smaller, so the library's fixed scratch is reused with its counters back at
zero.  Sizes beyond the scratch are rejected before any launch.
Every case prints its name and shapes (flushed) before its GPU work.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import workloads as wl
from harness import execute, gpu_pool, gpu_replay, oracle_pool, to_device
from oracle import attention as att
from test_gpu_parity import TOL, pba, say, small_workload  # noqa: F401

pytestmark = pytest.mark.gpu


def _prepared(w, device):
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    pool = gpu_pool(ex, device)
    gpu_replay(ex, pool, to_device(k_rows, w.shape.dtype, device),
               to_device(v_rows, w.shape.dtype, device))
    qb = wl.q_bits(w)
    q = to_device(qb, w.shape.dtype, device)
    tables = torch.from_numpy(ex.tables).to(device)
    lens = torch.from_numpy(ex.seq_lens).to(device)
    scale = 1.0 / math.sqrt(w.shape.head_dim)
    ref, ref_lse = att.paged_decode(opool, qb, list(ex.tables), ex.seq_lens, scale)
    torch.cuda.synchronize()
    return pool, q, tables, lens, scale, ref, ref_lse


def _check(pba, w, device, partition_tokens):
    say("noalloc", w.name, w.shape, "partition_tokens", partition_tokens)
    pool, q, tables, lens, scale, ref, ref_lse = _prepared(w, device)
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats(device)["allocation.all.allocated"]
    pba.paged_decode_noalloc(pool, q, tables, lens, scale, out=out, lse=lse,
                             partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats(device)["allocation.all.allocated"] == before
    need = pba.paged_decode_workspace_bytes(pool, Hq, B, tables.shape[1], partition_tokens)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=device)
    out_ws, lse_ws = pba.paged_decode(pool, q, tables, lens, scale, workspace=ws,
                                      partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ws) and torch.equal(lse, lse_ws), "differs from pba_paged_decode"
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    say("noalloc", w.name, "max abs err", err, "lse err", lerr, "workspace bytes", need)
    assert err <= TOL and lerr <= TOL
    return need


def test_noalloc_calls_in_a_row(pba, gpu):
    """Four calls: a split batch, a smaller one, the balanced decomposition,
    then a smaller split batch again (each layout's counters start where the
    previous call left them: at zero)."""
    big = small_workload("bf16", 64, 128, 8, 8, [4096, 3000, 4095, 1, 2500, 4096, 777, 2049],
                         20261202 + 4100)
    small = small_workload("bf16", 16, 128, 2, 4, [1, 15, 300, 1500, 2049], 20261202 + 4200)
    ragged = small_workload("bf16", 32, 64, 4, 2, [5, 900, 33, 2000, 64, 1], 20261202 + 4300)
    smaller = small_workload("bf16", 16, 64, 1, 1, [257, 40], 20261202 + 4400)
    needs = [_check(pba, big, gpu, 0), _check(pba, small, gpu, 256),
             _check(pba, ragged, gpu, -1), _check(pba, smaller, gpu, 256)]
    assert needs[0] > needs[1] > 0 and needs[2] > 0 and needs[1] > needs[3] > 0


def test_noalloc_rejects_beyond_scratch(pba, gpu):
    """Counter or state bytes beyond the fixed scratch: PBA_ERR_SCRATCH_LIMIT,
    nothing launched (the outputs keep their sentinel)."""
    say("noalloc limits")
    pool = pba.KVPool.empty(16, 16, 8, 128, torch.bfloat16, gpu)
    # 64 rows x 64 q-heads x 128 partitions of states (272 MB); then 40,000
    # rows x 8 kv heads in 2 partitions (1.28 MB of counters).
    for B, Hq, width, pt in ((64, 64, 2048, 256), (40000, 8, 32, 256)):
        q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device=gpu)
        tables = torch.zeros((B, width), dtype=torch.int32, device=gpu)
        lens = torch.ones(B, dtype=torch.int32, device=gpu)
        out = torch.full((B, Hq, 128), 7.0, dtype=torch.float32, device=gpu)
        with pytest.raises(pba.PBAError) as e:
            pba.paged_decode_noalloc(pool, q, tables, lens, out=out, want_lse=False,
                                     partition_tokens=pt)
        assert e.value.status == -11
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
    # The raw entry point: the same status through ctypes.
    st = pba._lib.pba_paged_decode_noalloc(pool._ref, q.data_ptr(), 8, tables.data_ptr(),
                                           32, lens.data_ptr(), 40000, ctypes.c_float(0.1),
                                           out.data_ptr(), None, 256, None)
    assert st == -11
