"""GPU parity of the shared-prefix decode (pba_paged_decode_shared) against the
binary64 oracle's monolithic decode, through the C ABI.

The plan comes from the caller-side helpers (blocks.sharing_order,
blocks.shared_plan) over block tables the oracle allocator produced; the
kernel must match the oracle within 2e-3 (bf16 inputs, fp32 accumulation),
agree with the plain decode, be deterministic, leave the workspace counters
at zero, and reject malformed plans in validate mode without writing.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from block_table_attention_amd.blocks import shared_plan, sharing_order
from harness import execute, gpu_pool, gpu_replay, oracle_pool, to_device
from oracle import attention as att

pytestmark = pytest.mark.gpu

TOL = 2e-3


def say(*msg):
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def pba(gpu):
    import block_table_attention_amd as m
    m.set_validate(True)
    yield m
    m.set_validate(False)


def prepare(w, device):
    """Run the script, build both pools, return the decode batch in sharing order."""
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    pool = gpu_pool(ex, device)
    gpu_replay(ex, pool, to_device(k_rows, w.shape.dtype, device),
               to_device(v_rows, w.shape.dtype, device))
    order = sharing_order(ex.tables)
    tables = np.ascontiguousarray(ex.tables[order])
    lens = np.ascontiguousarray(ex.seq_lens[order])
    qb = np.ascontiguousarray(wl.q_bits(w)[order])
    return opool, pool, tables, lens, qb


def run_shared(pba, w, device, pt=256, threshold=1, check_plain=True, tiles=4, packed=True):
    """packed=False drops the plan's private-range bound, so every private
    piece gets a work-group of its own; with it, ranges of at most 128
    positions go four rows per work-group."""
    say(w.name, w.shape, "seed", w.seed, "pt", pt, "threshold", threshold, "tiles", tiles,
        "packed", packed)
    opool, pool, tables, lens, qb = prepare(w, device)
    P, Hkv = w.shape.block_size, w.shape.num_kv_heads
    G = w.shape.num_q_heads // Hkv
    host = shared_plan(tables, lens, P, G, pt, threshold=threshold, tiles_per_item=tiles)
    if not packed:
        host.private_tokens = 0
    plan = pba.SharedPlan.from_host(host, device)
    q = to_device(qb, w.shape.dtype, device)
    tab = torch.from_numpy(tables).to(device)
    ln = torch.from_numpy(lens).to(device)
    scale = 1.0 / math.sqrt(w.shape.head_dim)
    out, lse = pba.paged_decode_shared(pool, q, tab, ln, plan, scale)
    torch.cuda.synchronize()
    ref, ref_lse = att.paged_decode(opool, qb, list(tables), lens, scale)
    err = np.max(np.abs(out.cpu().numpy() - ref))
    lerr = np.max(np.abs(lse.cpu().numpy() - ref_lse))
    say("   chunks", len(host.chunks), "items", host.items.shape[0], "max_slots", host.max_slots,
        "private_tokens", host.private_tokens, "max err", err, "lse err", lerr)
    assert err <= TOL and lerr <= TOL
    if check_plain:
        out2, _ = pba.paged_decode(pool, q, tab, ln, scale)
        torch.cuda.synchronize()
        assert torch.max(torch.abs(out2 - out)).item() <= TOL
    return out, lse, host


@pytest.mark.parametrize("packed", [True, False])
def test_shared_prefix_workload(pba, gpu, packed):
    """The full shared-prefix workload: 2000-token prefix over 128 rows, child
    and sibling suffixes shared in pairs, copy-on-write tails (private ranges
    of one block: packed four rows per work-group, or not)."""
    run_shared(pba, wl.shared_prefix(), gpu, packed=packed)


@pytest.mark.parametrize("G,P,d,batch", [(4, 16, 128, 6), (1, 64, 64, 5), (8, 32, 128, 7),
                                         (16, 16, 64, 3), (2, 256, 128, 9)])
def test_packed_private_ranges(pba, gpu, G, P, d, batch):
    """Private ranges of 1 to 128 positions, four rows per work-group: batches
    that leave the last group partly filled, rows whose only slot is the
    private one, rows with no private position, and tail chunks of every
    length."""
    rng = np.random.default_rng(20261202 + 7200 + G * 100 + P + batch)
    Hkv = 2
    w = wl.Workload(f"packed_g{G}_p{P}_d{d}", wl.Shape(P, G * Hkv, Hkv, d, "bf16", 512),
                    20261202 + 7200 + G)
    # Row 0 alone (its only slot is private); the others fork a common
    # prefix of whole blocks and add tokens of their own (none for the
    # first, 1..127 for the rest).
    w.actions = [("new",), ("prefill", 0, int(rng.integers(1, 129))),
                 ("new",), ("prefill", 1, 2 * P)]
    leaves = [0]
    for i in range(batch - 1):
        w.actions.append(("fork", 1))
        w.actions.append(("prefill", 2 + i, 0 if i == 0 else int(rng.integers(1, 128))))
        leaves.append(2 + i)
    w.decode = leaves
    _, _, host = run_shared(pba, w, gpu)
    assert 0 < host.private_tokens <= 128


@pytest.mark.parametrize("tiles", [1, 2, 4])
@pytest.mark.parametrize("G", [1, 4])
def test_tiles_per_item(pba, gpu, tiles, G):
    """Items of 1, 2 or 4 tiles (two-tile groups: one K/V load serves both
    tiles of a wave), full and partly filled last tiles."""
    w = wl.shared_prefix(children=13, prefix=900, lo=1, hi=300, num_blocks=1024)
    if G == 1:
        w.shape = wl.Shape(w.shape.block_size, w.shape.num_kv_heads, w.shape.num_kv_heads,
                           w.shape.head_dim, w.shape.dtype, w.shape.num_blocks)
    run_shared(pba, w, gpu, pt=512, tiles=tiles)


@pytest.mark.parametrize("pt", [256, 512, 2048])
def test_shared_prefix_partition_lengths(pba, gpu, pt):
    run_shared(pba, wl.shared_prefix(children=12, prefix=700, lo=1, hi=400, num_blocks=1024), gpu,
               pt=pt)


def _tree_workload(G, P, d, seed, depth=3, fan=3, num_blocks=2048):
    """A random fork tree: each level forks every leaf `fan` times and appends
    a random number of tokens (partial tails included)."""
    rng = np.random.default_rng(seed)
    Hkv = 2
    w = wl.Workload(f"tree_g{G}_p{P}_d{d}", wl.Shape(P, G * Hkv, Hkv, d, "bf16", num_blocks),
                    seed)
    w.actions = [("new",), ("prefill", 0, int(rng.integers(P, 6 * P)))]
    leaves = [0]
    nxt = 1
    for _ in range(depth):
        new = []
        for leaf in leaves:
            for _ in range(fan):
                w.actions.append(("fork", leaf))
                w.actions.append(("prefill", nxt, int(rng.integers(1, 4 * P))))
                new.append(nxt)
                nxt += 1
        leaves = new
    w.decode = leaves
    return w


@pytest.mark.parametrize("G,P,d", [(1, 16, 128), (2, 32, 64), (4, 64, 128), (8, 16, 128),
                                   (16, 256, 64), (3, 16, 128)])
def test_random_trees(pba, gpu, G, P, d):
    w = _tree_workload(G, P, d, seed=20261202 + 7000 + G * 10 + P)
    for thr in (1, 0):
        run_shared(pba, w, gpu, threshold=thr)
    run_shared(pba, w, gpu, packed=False)


def test_page_tree(pba, gpu):
    """The pages' four-sequence tree shape (0x0BB) with one kv head, G = 1."""
    w = wl.Workload("page_tree", wl.Shape(16, 1, 1, 128, "bf16", 64), 20261202 + 7100)
    w.actions = [("new",), ("prefill", 0, 32), ("fork", 0), ("fork", 0),
                 ("prefill", 1, 16), ("prefill", 2, 32),
                 ("fork", 1), ("fork", 1), ("fork", 2), ("fork", 2),
                 ("prefill", 3, 32), ("prefill", 4, 16), ("prefill", 5, 16), ("prefill", 6, 16)]
    w.decode = [3, 4, 5, 6]
    _, _, host = run_shared(pba, w, gpu)
    assert host.chunks == [(0, 4, 0, 32), (0, 2, 32, 48), (2, 4, 32, 64)]


def test_no_sharing_equals_plain(pba, gpu):
    """Without shared chunks the plan is all private pieces."""
    run_shared(pba, wl.lognormal(64, batch=48), gpu, pt=512)


def test_deterministic_and_counters_reset(pba, gpu):
    w = wl.shared_prefix(children=10, prefix=600, lo=3, hi=300, num_blocks=1024)
    opool, pool, tables, lens, qb = prepare(w, gpu)
    G = w.shape.num_q_heads // w.shape.num_kv_heads
    host = shared_plan(tables, lens, 16, G, 256)
    plan = pba.SharedPlan.from_host(host, gpu)
    q = to_device(qb, "bf16", gpu)
    tab = torch.from_numpy(tables).to(gpu)
    ln = torch.from_numpy(lens).to(gpu)
    B, Hq = qb.shape[0], qb.shape[1]
    need = pba.paged_decode_shared_workspace_bytes(pool, Hq, B, tables.shape[1], plan)
    ws = torch.zeros(need, dtype=torch.uint8, device=gpu)
    say("determinism", w.shape, "items", host.items.shape[0])
    outs = []
    for _ in range(3):
        out, lse = pba.paged_decode_shared(pool, q, tab, ln, plan, workspace=ws)
        torch.cuda.synchronize()
        outs.append((out.clone(), lse.clone()))
        assert torch.count_nonzero(ws[:4 * B * w.shape.num_kv_heads]).item() == 0
    assert all(torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1]) for o in outs)


def test_validate_mode_rejects_bad_plans(pba, gpu):
    """Malformed plans are rejected in validate mode and nothing is written."""
    w = wl.shared_prefix(children=4, prefix=64, lo=3, hi=40, num_blocks=128)
    opool, pool, tables, lens, qb = prepare(w, gpu)
    G = w.shape.num_q_heads // w.shape.num_kv_heads
    host = shared_plan(tables, lens, 16, G, 256)
    q = to_device(qb, "bf16", gpu)
    tab = torch.from_numpy(tables).to(gpu)
    ln = torch.from_numpy(lens).to(gpu)
    say("validate rejections", w.shape)

    def attempt(items, rowp, max_slots=host.max_slots):
        h = type(host)(items, rowp, max_slots, host.partition_tokens, host.chunks)
        plan = pba.SharedPlan.from_host(h, gpu)
        out = torch.full((qb.shape[0], qb.shape[1], qb.shape[2]), 7.0, device=gpu)
        with pytest.raises(pba.PBAError) as e:
            pba.paged_decode_shared(pool, q, tab, ln, plan, out=out)
        torch.cuda.synchronize()
        assert (out == 7.0).all()
        return e.value.status

    it, rp = host.items.copy(), host.row_private.copy()
    assert it.shape[0] > 0
    bad = it.copy(); bad[0, 3] += 16                       # piece past the chunk
    assert attempt(bad, rp) in (-6, -7)
    bad = it.copy(); bad[0, 4] = host.max_slots             # slot beyond the workspace
    assert attempt(bad, rp) == -6
    bad = rp.copy(); bad[0, 0] = 8                          # private start not aligned
    assert attempt(it, bad) == -6
    dup = np.concatenate([it, it[:1]])                      # a piece twice
    assert attempt(dup, rp) == -7
    bad = it.copy(); bad[0, 2] = -16
    assert attempt(bad, rp) == -6
    # A private-range bound below a row's private positions.
    assert host.private_tokens > 1
    h = type(host)(it, rp, host.max_slots, host.partition_tokens, host.chunks,
                   host.private_parts, host.private_tokens - 1)
    out = torch.full(qb.shape, 7.0, device=gpu)
    with pytest.raises(pba.PBAError) as e:
        pba.paged_decode_shared(pool, q, tab, ln, pba.SharedPlan.from_host(h, gpu), out=out)
    torch.cuda.synchronize()
    assert e.value.status == -6 and (out == 7.0).all()
    # A row whose table differs inside a chunk: swap in another row's tail id.
    assert tables[1, 0] == tables[0, 0]                    # both map the prefix's first block
    tab2 = tables.copy()
    tab2[1, 0] = (tables[0, 0] + 1) % w.shape.num_blocks
    h = pba.SharedPlan.from_host(host, gpu)
    with pytest.raises(pba.PBAError):
        pba.paged_decode_shared(pool, q, torch.from_numpy(tab2).to(gpu), ln, h)
