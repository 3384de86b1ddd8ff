"""GPU parity of the balanced decode (partition_tokens = PBA_PARTITIONS_BALANCED):
the batch's 32-token chunks split evenly over one work-group per CU, pieces of
cut rows merged by work-group and across work-groups.

* Every small shape (P, d, G; fp32 pools fall back to the grid), the workload
  batches, and the long-context workloads at full size (every (request, kv head) pair) match
  the binary64 oracle within 2e-3.
* Edge cases: one row of one token; fewer chunks than waves; 2048 rows (the
  largest balanced batch); rows much longer than a work-group's range.
* Dense, compact (ragged) and contiguous-slot tables give bitwise the same
  result (same chunks, same order); repeated calls are bitwise equal and leave
  the workspace counters at zero; the result agrees with the grid decode.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from harness import execute, gpu_pool, gpu_replay, oracle_pool, to_device
from oracle import attention as att
from oracle import views
from test_gpu_parity import SMALL, pba, run_workload, small_workload  # noqa: F401

pytestmark = pytest.mark.gpu

BAL = -1
TOL = 2e-3


def say(*msg):
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_shapes_balanced(pba, gpu, case):
    dtype, P, d, Hkv, G, lengths = SMALL[case]
    w = small_workload(dtype, P, d, Hkv, G, lengths, 20261202 + 1000 + case)
    run_workload(pba, w, gpu, partition_tokens=BAL)


@pytest.mark.parametrize("make", [wl.batch32, wl.shared_prefix, lambda: wl.lognormal(16),
                                  lambda: wl.lognormal(64), lambda: wl.lognormal(256)])
def test_workloads_balanced(pba, gpu, make):
    run_workload(pba, make(), gpu, partition_tokens=BAL)


def test_long16k_balanced_all_pairs(pba, gpu):
    run_workload(pba, wl.long16k(), gpu, partition_tokens=BAL)


def test_long64k_balanced_all_pairs(pba, gpu):
    run_workload(pba, wl.long64k(), gpu, partition_tokens=BAL)


def test_single_token_row(pba, gpu):
    w = small_workload("bf16", 16, 128, 1, 4, [1], 20261202 + 1500)
    run_workload(pba, w, gpu, partition_tokens=BAL)


def test_max_batch_of_short_rows(pba, gpu):
    """2048 rows of 1..90 tokens, two kv heads: most rows inside one wave,
    some cut at wave and work-group boundaries."""
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 91, size=2048)]
    w = small_workload("bf16", 16, 64, 2, 2, lengths, 20261202 + 1600)
    run_workload(pba, w, gpu, check_pool=False, partition_tokens=BAL)


def _prepare(w, device):
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    pool = gpu_pool(ex, device)
    gpu_replay(ex, pool, to_device(k_rows, w.shape.dtype, device),
               to_device(v_rows, w.shape.dtype, device))
    return ex, opool, pool


def test_table_encodings_agree_and_repeat(pba, gpu):
    w = wl.lognormal(16, batch=96)
    ex, opool, pool = _prepare(w, gpu)
    say("balanced encodings", w.shape)
    q = to_device(wl.q_bits(w), "bf16", gpu)
    tab = torch.from_numpy(ex.tables).to(gpu)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    B, Hq, d = q.shape
    need = pba.paged_decode_workspace_bytes(pool, Hq, B, tab.shape[1], BAL)
    ws = torch.zeros(need, dtype=torch.uint8, device=gpu)
    outs = []
    for _ in range(3):
        out, lse = pba.paged_decode(pool, q, tab, lens, partition_tokens=BAL, workspace=ws)
        torch.cuda.synchronize()
        outs.append((out.clone(), lse.clone()))
        assert torch.count_nonzero(ws[:4 * B * pool.num_kv_heads]).item() == 0
    assert all(torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1]) for o in outs)
    entries, offsets = views.pack_ragged(ex.tables, ex.seq_lens, 16)
    out_r, lse_r = pba.paged_decode_ragged(pool, q, torch.from_numpy(entries).to(gpu),
                                           torch.from_numpy(offsets).to(gpu), lens, tab.shape[1],
                                           partition_tokens=BAL)
    torch.cuda.synchronize()
    assert torch.equal(out_r, outs[0][0]) and torch.equal(lse_r, outs[0][1])
    out_g, _ = pba.paged_decode(pool, q, tab, lens, partition_tokens=0)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(out_g - outs[0][0])).item() <= 1e-5


def test_contiguous_slots_balanced(pba, gpu):
    """Slot-indexed decode over a plain buffer laid out as contiguous slots:
    balanced equals the grid within 1e-5 and the oracle within 2e-3."""
    H, G, d, P = 2, 4, 128, 16
    lens = np.array([700, 3, 129, 1500, 64, 1, 999], dtype=np.int32)
    B = len(lens)
    bps = int(-(-lens.max() // P))
    say("contiguous balanced", lens.tolist())
    kb = wl.normal_bits(20261202 + 1700, (B * bps, H, P, d), "bf16")
    vb = wl.normal_bits(20261202 + 1701, (B * bps, H, d, P), "bf16")
    pool = pba.KVPool(to_device(kb, "bf16", gpu), to_device(vb, "bf16", gpu))
    slot = np.array([6, 0, 3, 5, 1, 2, 4], dtype=np.int32)
    qb = wl.normal_bits(20261202 + 1702, (B, H * G, d), "bf16")
    q = to_device(qb, "bf16", gpu)
    si = torch.from_numpy(slot).to(gpu)
    ln = torch.from_numpy(lens).to(gpu)
    out_b, lse_b = pba.paged_decode_contiguous(pool, q, si, bps, ln, partition_tokens=BAL)
    out_g, _ = pba.paged_decode_contiguous(pool, q, si, bps, ln, partition_tokens=0)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(out_b - out_g)).item() <= 1e-5
    from oracle.pool import BitPool
    opool = BitPool(kb, vb, "bf16")
    tables = [[int(s) * bps + j for j in range(bps)] for s in slot]
    ref, ref_lse = att.paged_decode(opool, qb, tables, lens, 1 / math.sqrt(d))
    assert np.max(np.abs(out_b.cpu().numpy() - ref)) <= TOL
    assert np.max(np.abs(lse_b.cpu().numpy() - ref_lse)) <= TOL


@pytest.mark.parametrize("P,d,P_k", [(64, 128, None), (128, 64, None), (256, 128, None),
                                     (256, 128, 64)])
def test_chunk_pairs(pba, gpu, P, d, P_k):
    """Blocks of 64 tokens or more: a wave that prefetches an even chunk also
    loads its odd partner's V (same block).  Hundreds of ragged rows put wave
    and work-group boundaries on odd and even chunks, next to rows with odd
    chunk counts and short tails; balanced equals the grid within 1e-5 and the
    oracle within 2e-3, also through a 64-token kernel view of 256-token tiles."""
    rng = np.random.default_rng(4000 + P + d)
    lengths = [int(x) for x in rng.integers(1, 420, size=320)]
    w = small_workload("bf16", P, d, 2, 4, lengths, 20261202 + 1800 + P + d)
    ex, opool, pool = _prepare(w, gpu)
    say("chunk pairs", w.shape, "kernel block", P_k)
    qb = wl.q_bits(w)
    q = to_device(qb, "bf16", gpu)
    tab = torch.from_numpy(ex.tables).to(gpu)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    if P_k is not None:
        pool = pool.kernel_view(P_k)
        tab = pba.expand_block_tables(tab, pool.split_log2)
    out_b, lse_b = pba.paged_decode(pool, q, tab, lens, partition_tokens=BAL)
    out_g, lse_g = pba.paged_decode(pool, q, tab, lens, partition_tokens=0)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(out_b - out_g)).item() <= 1e-5
    assert torch.max(torch.abs(lse_b - lse_g)).item() <= 1e-5
    ref, ref_lse = att.paged_decode(opool, qb, list(ex.tables), ex.seq_lens, 1 / math.sqrt(d))
    assert np.max(np.abs(out_b.cpu().numpy() - ref)) <= TOL
    assert np.max(np.abs(lse_b.cpu().numpy() - ref_lse)) <= TOL


@pytest.mark.parametrize("G,d", [(16, 64), (2, 128)])
def test_group_sizes(pba, gpu, G, d):
    """The widest LDS pieces the balanced decode takes (G = 16 at head_dim 64,
    8 wave pieces of 16 x 66 floats) and a narrow group, on ragged rows."""
    rng = np.random.default_rng(4100 + G)
    lengths = [int(x) for x in rng.integers(1, 600, size=150)]
    w = small_workload("bf16", 16, d, 2, G, lengths, 20261202 + 1900 + G)
    plan = pba.paged_decode_plan(pba.KVPool.empty(8, 16, 2, d, torch.bfloat16, gpu), 2 * G, 150,
                                 40, BAL)
    assert plan[0] == 0  # served by the balanced decode, not the grid
    run_workload(pba, w, gpu, partition_tokens=BAL)
