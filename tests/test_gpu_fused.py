"""GPU parity of the fused decode step (pba_paged_decode_append): each row's
new token appended and the batch decoded in one call.

* Against the separate calls (kv_append, then paged_decode) on a second copy
  of the pool: the pools bit for bit, out and lse bit for bit.
* Against the oracle: the pool bit for bit (after every append of the
  workload), the decode within 2e-3.
* Shapes: block sizes 16-256, head_dim 64 and 128, G 1-16, partitions of the
  library plan, 256 and 512 tokens and the balanced decomposition, fp32 pools
  (every one of them appends in the decode launch), rows that append
  nothing, rows whose new token falls in a wave's first chunk, kernel views
  of an allocator pool, the balanced decomposition over hundreds of short
  rows, and the 8 x 16,384-token workload at full size.
* Validate mode rejects a slot that is not the row's last position, and a
  new token in a block another row references, with nothing written.
Every case prints its name, shapes and seed (flushed) before its GPU work.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from harness import execute, gpu_pool, gpu_replay, oracle_pool, to_bits, to_device
from oracle import attention as att
from test_gpu_parity import TOL, pba, say  # noqa: F401

pytestmark = pytest.mark.gpu


def step_workload(dtype, P, d, Hkv, G, lengths, appends, seed):
    """Rows prefilled to length - appends[r], then one appended token for each
    row with appends[r] == 1 (in row order): the step's new tokens."""
    nb = sum(-(-T // P) for T in lengths) + 9
    w = wl.Workload(f"step_{dtype}_P{P}_d{d}_G{G}", wl.Shape(P, Hkv * G, Hkv, d, dtype, nb), seed)
    for r, (T, a) in enumerate(zip(lengths, appends)):
        w.actions.append(("new",))
        w.actions.append(("prefill", r, T - a))
    for r, a in enumerate(appends):
        if a:
            w.actions.append(("append", r))
    w.decode = list(range(len(lengths)))
    return w


def split_step(ex, n_new):
    """The workload's trace without its last n_new writes (the step's new
    tokens, one per appending row in row order), and those writes as one
    append op."""
    last = ex.ops[-1]
    assert last[0] == "append" and len(last[1]) >= n_new
    ops = list(ex.ops[:-1])
    if len(last[1]) > n_new:
        ops.append(("append", last[1][:-n_new], last[2], last[3] - n_new))
    step = ("append", last[1][-n_new:], last[3] - n_new, last[3])
    return type(ex)(ex.workload, ex.alloc, ops, ex.tables, ex.seq_lens, ex.n_writes), step


def run_fused(pba, w, device, appends, partition_tokens=0, kernel_block=None):
    say(w.name, w.shape, "seed", w.seed, "partition_tokens", partition_tokens,
        "kernel_block", kernel_block)
    ex = execute(w)
    prefix, last = split_step(ex, sum(appends))
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    dt = w.shape.dtype
    kd, vd = to_device(k_rows, dt, device), to_device(v_rows, dt, device)
    pools = []
    for _ in range(2):
        pool = gpu_pool(ex, device)
        gpu_replay(prefix, pool, kd, vd)
        pools.append(pool)
    B = len(w.decode)
    Hkv, D = w.shape.num_kv_heads, w.shape.head_dim
    rows_appending = [r for r in range(B) if appends[r]]
    new_slots = np.full(B, -1, dtype=np.int64)
    new_slots[rows_appending] = last[1]
    knew = torch.zeros((B, Hkv, D), dtype=kd.dtype, device=device)
    vnew = torch.zeros_like(knew)
    idx = torch.tensor(rows_appending, dtype=torch.int64, device=device)
    knew[idx] = kd[last[2]:last[3]]
    vnew[idx] = vd[last[2]:last[3]]
    qb = wl.q_bits(w)
    q = to_device(qb, dt, device)
    tables = torch.from_numpy(ex.tables).to(device)
    lens = torch.from_numpy(ex.seq_lens).to(device)
    slots_d = torch.from_numpy(new_slots).to(device)
    scale = 1.0 / math.sqrt(D)
    fp, sp = pools
    if kernel_block:
        fp, sp = fp.kernel_view(kernel_block), sp.kernel_view(kernel_block)
        tables = pba.expand_block_tables(tables, fp.split_log2)
    out, lse = pba.paged_decode_append(fp, slots_d, knew, vnew, q, tables, lens, scale,
                                       partition_tokens=partition_tokens)
    pba.kv_append(pools[1], torch.from_numpy(last[1]).to(device), kd[last[2]:last[3]],
                  vd[last[2]:last[3]])
    out2, lse2 = pba.paged_decode(sp, q, tables, lens, scale, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(pools[0].k), opool.k), "K pool bits differ from the oracle"
    assert np.array_equal(to_bits(pools[0].v), opool.v), "V pool bits differ from the oracle"
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "fused differs from separate calls"
    ref, ref_lse = att.paged_decode(opool, qb, list(ex.tables), ex.seq_lens, scale)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    say(w.name, "max abs err", err, "lse err", lerr)
    assert err <= TOL and lerr <= TOL
    return ex, pools[0]


CASES = [
    # (dtype, P, d, Hkv, G, lengths)
    ("bf16", 16, 128, 2, 4, [1, 2, 17, 33, 300, 1500, 2049]),
    ("bf16", 32, 128, 1, 8, [32, 64, 65, 700, 1025]),
    ("bf16", 64, 64, 2, 1, [2, 63, 64, 129, 1000]),
    ("bf16", 128, 128, 3, 16, [5, 128, 257, 600]),
    ("bf16", 256, 64, 1, 2, [255, 256, 257, 1300]),
    ("f32", 16, 64, 1, 1, [35, 2, 16, 17]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("partition_tokens", [0, 256, -1])
def test_fused_step_matches_separate_calls(pba, gpu, case, partition_tokens):
    dtype, P, d, Hkv, G, lengths = CASES[case]
    appends = [1 if (r % 3) != 1 else 0 for r in range(len(lengths))]
    appends[0] = 1
    w = step_workload(dtype, P, d, Hkv, G, lengths, appends, 20261202 + 5000 + case)
    run_fused(pba, w, gpu, appends, partition_tokens)


@pytest.mark.parametrize("P,rows,longest", [(16, 400, 300), (64, 1200, 120), (256, 400, 300),
                                             (64, 400, 300)])
def test_fused_step_balanced_many_segments(pba, gpu, P, rows, longest):
    """The balanced decomposition with the appends in its launch: hundreds of
    rows of 1 to a few hundred tokens, so waves cross many (request, kv head)
    segments, start and end inside them, and (P >= 64) meet last chunks of
    both parities behind paired V loads; two rows in three append."""
    rng = np.random.default_rng(20261202 + 5300 + P + rows)
    lengths = [int(x) for x in rng.integers(1, longest + 1, size=rows)]
    appends = [1 if r % 3 else 0 for r in range(rows)]
    for r, T in enumerate(lengths):
        if T == 1:
            appends[r] = 1          # a row whose only token is the step's
    w = step_workload("bf16", P, 128, 2, 4, lengths, appends, 20261202 + 5300 + P + rows)
    run_fused(pba, w, gpu, appends, -1)


@pytest.mark.parametrize("partition_tokens", [512, -1])
def test_fused_step_kernel_view(pba, gpu, partition_tokens):
    """A 64-token allocator pool read as 16-token kernel blocks, with
    partitions and with the balanced decomposition: the new token's slot is
    the same in both views."""
    lengths = [3, 64, 65, 700, 1500]
    appends = [1] * len(lengths)
    w = step_workload("bf16", 64, 128, 2, 4, lengths, appends, 20261202 + 5100)
    run_fused(pba, w, gpu, appends, partition_tokens, kernel_block=16)


def test_fused_step_long16k(pba, gpu):
    """8 x 16,384 tokens (16,383 prefilled, the step's token appended by the
    decode launch), 4 partitions of 4096: every pair against the oracle."""
    w = wl.long16k()
    run_fused(pba, w, gpu, [1] * 8, 0)


def test_fused_step_validate_rejects(pba, gpu):
    lengths = [40, 100, 17]
    appends = [1, 1, 1]
    w = step_workload("bf16", 16, 64, 1, 2, lengths, appends, 20261202 + 5200)
    say("fused validate", w.shape)
    ex = execute(w)
    prefix, last = split_step(ex, 3)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    kd, vd = to_device(k_rows, "bf16", gpu), to_device(v_rows, "bf16", gpu)
    pool = gpu_pool(ex, gpu)
    gpu_replay(prefix, pool, kd, vd)
    torch.cuda.synchronize()
    kb, vb = pool.k.clone(), pool.v.clone()
    q = to_device(wl.q_bits(w), "bf16", gpu)
    tables = torch.from_numpy(ex.tables).to(gpu)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    knew, vnew = kd[last[2]:last[3]].contiguous(), vd[last[2]:last[3]].contiguous()
    good = last[1].copy()
    for bad, status in ((np.array([good[0] - 1, good[1], good[2]]), -6),   # position T - 2
                        (np.array([good[0], good[2], good[2]]), -6)):      # another row's slot
        with pytest.raises(pba.PBAError) as e:
            pba.paged_decode_append(pool, torch.from_numpy(bad).to(gpu), knew, vnew, q, tables,
                                    lens)
        assert e.value.status == status
        torch.cuda.synchronize()
        assert torch.equal(pool.k.view(torch.int16), kb.view(torch.int16))
        assert torch.equal(pool.v.view(torch.int16), vb.view(torch.int16))
    # Row 1's table made to reference row 0's last block: row 0's new token
    # would be visible to row 1 (a shared block is copied before a write).
    shared = ex.tables.copy()
    shared[1][0] = shared[0][(lengths[0] - 1) // 16]
    with pytest.raises(pba.PBAError) as e:
        pba.paged_decode_append(pool, torch.from_numpy(good).to(gpu), knew, vnew, q,
                                torch.from_numpy(shared).to(gpu), lens)
    assert e.value.status == -7
    torch.cuda.synchronize()
    assert torch.equal(pool.k.view(torch.int16), kb.view(torch.int16))
    assert torch.equal(pool.v.view(torch.int16), vb.view(torch.int16))
