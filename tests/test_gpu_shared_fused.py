"""GPU parity of the fused shared-prefix decode step
(pba_paged_decode_shared_append): each row's new token appended and the
batch decoded through a shared-prefix plan in one call.

* Against the separate calls (kv_append, then paged_decode_shared) on a
  second copy of the pool: the pools bit for bit, out and lse bit for bit.
* Against the oracle: the pool bit for bit, the decode within 2e-3.
* Plans: packed private ranges (four rows per work-group) and private pieces
  (a work-group per piece, the token in a row's last piece at any of its
  waves' chunks); rows that append nothing.
* Validate mode rejects a slot that is not the row's last position, and one
  whose position lies in a shared chunk, with nothing written.
Every case prints its name, shapes and seed (flushed) before its GPU work."""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from block_table_attention_amd.blocks import shared_plan, sharing_order
from harness import execute, gpu_pool, gpu_replay, oracle_pool, to_bits, to_device
from oracle import attention as att
from test_gpu_fused import split_step
from test_gpu_shared import TOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pba(gpu):
    import block_table_attention_amd as m
    m.set_validate(True)
    yield m
    m.set_validate(False)


def step_on(w, appending):
    """The workload plus one appended token for each leaf in `appending`
    (their private tails or fresh blocks: no copy-on-write in the step)."""
    for r in appending:
        w.actions.append(("append", r))
    return w


def prepare(w, appending, device):
    ex = execute(w)
    prefix, last = split_step(ex, len(appending))
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    dt = w.shape.dtype
    kd, vd = to_device(k_rows, dt, device), to_device(v_rows, dt, device)
    pools = []
    for _ in range(2):
        pool = gpu_pool(ex, device)
        gpu_replay(prefix, pool, kd, vd)
        pools.append(pool)
    return ex, last, opool, kd, vd, pools


def run_case(pba, w, device, appending, pt=256, tiles=2, packed=True):
    say(w.name, w.shape, "seed", w.seed, "pt", pt, "tiles", tiles, "packed", packed,
        "appending", len(appending))
    ex, last, opool, kd, vd, (fp, sp) = prepare(w, appending, device)
    B = len(w.decode)
    P, Hkv, D = w.shape.block_size, w.shape.num_kv_heads, w.shape.head_dim
    G = w.shape.num_q_heads // Hkv
    order = sharing_order(ex.tables)
    tables = np.ascontiguousarray(ex.tables[order])
    lens = np.ascontiguousarray(ex.seq_lens[order])
    host = shared_plan(tables, lens, P, G, pt, tiles_per_item=tiles)
    if not packed:
        host.private_tokens = 0
    plan = pba.SharedPlan.from_host(host, device)
    # The step's tokens in decode-row order, then in sharing order.
    rows = [w.decode.index(r) for r in appending]
    new_slots = np.full(B, -1, dtype=np.int64)
    new_slots[rows] = last[1]
    knew = torch.zeros((B, Hkv, D), dtype=kd.dtype, device=device)
    vnew = torch.zeros_like(knew)
    idx = torch.tensor(rows, dtype=torch.int64, device=device)
    knew[idx] = kd[last[2]:last[3]]
    vnew[idx] = vd[last[2]:last[3]]
    perm = torch.from_numpy(order).to(device)
    qb = np.ascontiguousarray(wl.q_bits(w)[order])
    q = to_device(qb, w.shape.dtype, device)
    tab = torch.from_numpy(tables).to(device)
    ln = torch.from_numpy(lens).to(device)
    scale = 1.0 / math.sqrt(D)
    out, lse = pba.paged_decode_shared_append(fp, torch.from_numpy(new_slots[order]).to(device),
                                              knew[perm].contiguous(), vnew[perm].contiguous(), q,
                                              tab, ln, plan, scale)
    pba.kv_append(sp, torch.from_numpy(last[1]).to(device), kd[last[2]:last[3]],
                  vd[last[2]:last[3]])
    out2, lse2 = pba.paged_decode_shared(sp, q, tab, ln, plan, scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(fp.k), opool.k), "K pool bits differ from the oracle"
    assert np.array_equal(to_bits(fp.v), opool.v), "V pool bits differ from the oracle"
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "fused differs from separate calls"
    ref, ref_lse = att.paged_decode(opool, qb, list(tables), lens, scale)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    say(w.name, "items", host.items.shape[0], "max err", err, "lse err", lerr)
    assert err <= TOL and lerr <= TOL
    return host, ex, fp, new_slots, order, knew, vnew, q, tab, ln, plan


@pytest.mark.parametrize("packed", [True, False])
def test_fused_shared_prefix_step(pba, gpu, packed):
    """The shared-prefix workload with one more token on every row (private
    tails of 1-16 positions: four rows per work-group, or a piece each)."""
    w = wl.shared_prefix(children=16, prefix=1000, lo=1, hi=300, num_blocks=2048)
    run_case(pba, step_on(w, list(w.decode)), gpu, list(w.decode), pt=512, packed=packed)


@pytest.mark.parametrize("G,P,d", [(4, 16, 128), (8, 32, 64), (1, 64, 128), (2, 256, 64),
                                   (16, 16, 128)])
def test_fused_long_private_ranges(pba, gpu, G, P, d):
    """Private ranges of several 256-position pieces (no packing): the new
    token lies in a row's last piece, in the chunk of any of its four waves;
    every other row appends nothing."""
    rng = np.random.default_rng(20261202 + 9600 + G * 10 + P)
    Hkv = 2
    w = wl.Workload(f"fused_long_g{G}_p{P}_d{d}", wl.Shape(P, G * Hkv, Hkv, d, "bf16", 1024),
                    20261202 + 9600 + G)
    w.actions = [("new",), ("prefill", 0, 2 * P)]
    leaves = []
    for i in range(6):
        w.actions.append(("fork", 0))
        w.actions.append(("prefill", 1 + i, int(rng.integers(300, 900))))
        leaves.append(1 + i)
    w.decode = leaves
    run_case(pba, step_on(w, leaves[::2]), gpu, leaves[::2], pt=256, packed=False)


def _edge_workload(P, G, d, seed):
    """Two forks of a two-block prefix (5 and 40 tokens of their own), and
    three rows of their own: empty, P - 1 and P tokens before the step."""
    Hkv = 2
    w = wl.Workload(f"fused_edges_g{G}_p{P}_d{d}", wl.Shape(P, G * Hkv, Hkv, d, "bf16", 256), seed)
    w.actions = [("new",), ("prefill", 0, 2 * P), ("fork", 0), ("fork", 0), ("release", 0),
                 ("prefill", 1, 5), ("prefill", 2, 40),
                 ("new",), ("prefill", 3, 0), ("new",), ("prefill", 4, P - 1),
                 ("new",), ("prefill", 5, P)]
    w.decode = [1, 2, 3, 4, 5]
    return w


@pytest.mark.parametrize("packed", [True, False])
@pytest.mark.parametrize("tiles", [1, 2])
@pytest.mark.parametrize("G,P,d", [(4, 16, 128), (2, 64, 64)])
def test_fused_shared_edges(pba, gpu, packed, tiles, G, P, d):
    """A row whose only position is the new token (T = 1), a new token at a
    block's last offset (T = P) and at a fresh block's first (T = P + 1), a
    shared-prefix row that appends and one that does not."""
    w = _edge_workload(P, G, d, 20261202 + 9800 + G + P)
    appending = [3, 4, 5, 2]
    run_case(pba, step_on(w, appending), gpu, appending, pt=256, tiles=tiles, packed=packed)


def test_fused_shared_no_new_tokens(pba, gpu):
    """Every new slot negative: the pool is untouched and out / lse equal
    paged_decode_shared's bit for bit."""
    w = step_on(_edge_workload(16, 4, 128, 20261202 + 9900), [3, 4, 5, 2])
    say(w.name, w.shape, "seed", w.seed, "no new tokens")
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    pool = gpu_pool(ex, gpu)
    gpu_replay(ex, pool, to_device(k_rows, "bf16", gpu), to_device(v_rows, "bf16", gpu))
    order = sharing_order(ex.tables)
    tables = np.ascontiguousarray(ex.tables[order])
    lens = np.ascontiguousarray(ex.seq_lens[order])
    plan = pba.SharedPlan.from_host(shared_plan(tables, lens, 16, 4, 256, tiles_per_item=2), gpu)
    B = len(w.decode)
    q = to_device(np.ascontiguousarray(wl.q_bits(w)[order]), "bf16", gpu)
    tab, ln = torch.from_numpy(tables).to(gpu), torch.from_numpy(lens).to(gpu)
    none = torch.full((B,), -1, dtype=torch.int64, device=gpu)
    kn = torch.zeros((B, 2, 128), dtype=torch.bfloat16, device=gpu)
    kb, vb = pool.k.clone(), pool.v.clone()
    out, lse = pba.paged_decode_shared_append(pool, none, kn, kn, q, tab, ln, plan)
    out2, lse2 = pba.paged_decode_shared(pool, q, tab, ln, plan)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    assert torch.equal(pool.k.view(torch.int16), kb.view(torch.int16))
    assert torch.equal(pool.v.view(torch.int16), vb.view(torch.int16))


def test_fused_shared_validate_rejects(pba, gpu):
    """A slot at T - 2 is rejected, and so is a new token in a block another
    row references; the pool is left untouched."""
    w = wl.shared_prefix(children=4, prefix=160, lo=1, hi=40, num_blocks=256)
    w = step_on(w, list(w.decode))
    host, ex, fp, new_slots, order, knew, vnew, q, tab, ln, plan = run_case(pba, w, gpu,
                                                                            list(w.decode))
    say("fused shared validate: slot at T - 2")
    kb, vb = fp.k.clone(), fp.v.clone()
    ns = new_slots[order].copy()
    r = int(np.argmax(ns >= 0))
    bad = ns.copy()
    bad[r] -= 1
    with pytest.raises(pba.PBAError) as e:
        pba.paged_decode_shared_append(fp, torch.from_numpy(bad).to(gpu), knew, vnew, q, tab, ln,
                                       plan)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert torch.equal(fp.k.view(torch.int16), kb.view(torch.int16))
    assert torch.equal(fp.v.view(torch.int16), vb.view(torch.int16))

    # Two rows with one table (a fork that has not written yet): with a
    # partial last block the block is read privately by both rows (writing it
    # needs a copy first: PBA_ERR_OVERLAP); with whole blocks it is a chunk's
    # (outside the private range: PBA_ERR_OUT_OF_RANGE).
    P, Hkv, D = 16, 2, 64
    for length, status in ((3 * P + 5, -7), (4 * P, -6)):
        say("fused shared validate: twins of length", length)
        w2 = wl.Workload("fused_shared_twins", wl.Shape(P, 4 * Hkv, Hkv, D, "bf16", 64),
                         20261202 + 9700)
        w2.actions = [("new",), ("prefill", 0, length), ("fork", 0), ("fork", 0),
                      ("prefill", 2, 9)]
        w2.decode = [0, 1, 2]
        ex2 = execute(w2)
        k_rows, v_rows = wl.kv_rows(w2, ex2.n_writes)
        pool = gpu_pool(ex2, gpu)
        gpu_replay(ex2, pool, to_device(k_rows, "bf16", gpu), to_device(v_rows, "bf16", gpu))
        order2 = sharing_order(ex2.tables)
        tables = np.ascontiguousarray(ex2.tables[order2])
        lens = np.ascontiguousarray(ex2.seq_lens[order2])
        plan2 = pba.SharedPlan.from_host(shared_plan(tables, lens, P, 4, 256, tiles_per_item=2),
                                         gpu)
        t0 = next(i for i in range(3) for j in range(3)
                  if i != j and lens[i] == lens[j] and (tables[i] == tables[j]).all())
        T = int(lens[t0])
        ns2 = np.full(3, -1, dtype=np.int64)
        ns2[t0] = int(tables[t0][(T - 1) // P]) * P + (T - 1) % P
        kn = torch.zeros((3, Hkv, D), dtype=torch.bfloat16, device=gpu)
        q2 = torch.zeros((3, 4 * Hkv, D), dtype=torch.bfloat16, device=gpu)
        kb, vb = pool.k.clone(), pool.v.clone()
        with pytest.raises(pba.PBAError) as e:
            pba.paged_decode_shared_append(pool, torch.from_numpy(ns2).to(gpu), kn, kn, q2,
                                           torch.from_numpy(tables).to(gpu),
                                           torch.from_numpy(lens).to(gpu), plan2)
        assert e.value.status == status
        torch.cuda.synchronize()
        assert torch.equal(pool.k.view(torch.int16), kb.view(torch.int16))
        assert torch.equal(pool.v.view(torch.int16), vb.view(torch.int16))


def test_fused_shared_graph_replay(pba, gpu):
    """The shared-prefix step (block_copy of the copy-on-write pairs, then
    paged_decode_shared_append) captured in a HIP graph: every replay, with
    eager calls and synchronisations between replays, equals the eager step
    bit for bit (pool bytes, out, lse) and leaves the counters at zero; the
    result matches the oracle."""
    import bench

    w = wl.shared_prefix(children=6, prefix=300, lo=3, hi=40, num_blocks=160)
    say("fused shared graph replay", w.shape, "seed", w.seed)
    plan = bench.plan_script(w)
    assert len(plan.step_src) > 0 and len(plan.step_slots) == 6
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    kd, vd = to_device(k_rows, "bf16", gpu), to_device(v_rows, "bf16", gpu)
    k0, v0 = wl.pool_poison(w)
    pools = [pba.KVPool(to_device(k0, "bf16", gpu), to_device(v0, "bf16", gpu)) for _ in range(2)]
    for pool in pools:
        for op in plan.setup:
            if op[0] == "copy":
                pba.block_copy(pool, torch.from_numpy(op[1]).to(gpu), torch.from_numpy(op[2]).to(gpu))
            else:
                pba.kv_append(pool, torch.from_numpy(op[1]).to(gpu), kd[op[2]:op[3]], vd[op[2]:op[3]])
    P, Hkv, D = w.shape.block_size, w.shape.num_kv_heads, w.shape.head_dim
    Hq = w.shape.num_q_heads
    order = sharing_order(plan.tables)
    tables = np.ascontiguousarray(plan.tables[order])
    lens = np.ascontiguousarray(plan.seq_lens[order])
    B = len(lens)
    splan = pba.SharedPlan.from_host(shared_plan(tables, lens, P, Hq // Hkv, 256,
                                                 tiles_per_item=2), gpu)
    # Row (sharing order) of each new token: the row whose last position it is.
    last = {int(tables[r, (T - 1) // P]) * P + (T - 1) % P: r for r, T in enumerate(lens)}
    rows = [last[int(s)] for s in plan.step_slots]
    ns = np.full(B, -1, dtype=np.int64)
    ns[rows] = plan.step_slots
    lo, hi = plan.step_rows
    knew = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device=gpu)
    vnew = torch.zeros_like(knew)
    idx = torch.tensor(rows, dtype=torch.int64, device=gpu)
    knew[idx] = kd[lo:hi]
    vnew[idx] = vd[lo:hi]
    new_slots = torch.from_numpy(ns).to(gpu)
    src = torch.from_numpy(plan.step_src).to(gpu)
    dst = torch.from_numpy(plan.step_dst).to(gpu)
    qb = np.ascontiguousarray(wl.q_bits(w)[order])
    q = to_device(qb, "bf16", gpu)
    tab, ln = torch.from_numpy(tables).to(gpu), torch.from_numpy(lens).to(gpu)
    ws_bytes = pba.paged_decode_shared_workspace_bytes(pools[0], Hq, B, tables.shape[1], splan)
    assert ws_bytes > 0
    bufs = [dict(out=torch.empty((B, Hq, D), dtype=torch.float32, device=gpu),
                 lse=torch.empty((B, Hq), dtype=torch.float32, device=gpu),
                 ws=torch.zeros(ws_bytes, dtype=torch.uint8, device=gpu)) for _ in range(2)]

    def step(pool, b):
        pba.block_copy(pool, src, dst)
        pba.paged_decode_shared_append(pool, new_slots, knew, vnew, q, tab, ln, splan,
                                       out=b["out"], lse=b["lse"], workspace=b["ws"])

    step(pools[0], bufs[0])                    # eager reference, validated
    torch.cuda.synchronize()
    pba.set_validate(False)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(pools[1], bufs[1])            # warm the graph's buffers once
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(pools[1], bufs[1])
        for rep in range(3):
            bufs[1]["out"].fill_(float("nan"))
            bufs[1]["lse"].fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(bufs[1]["out"], bufs[0]["out"]), rep
            assert torch.equal(bufs[1]["lse"], bufs[0]["lse"]), rep
            assert torch.equal(pools[1].k.view(torch.int16), pools[0].k.view(torch.int16)), rep
            assert torch.equal(pools[1].v.view(torch.int16), pools[0].v.view(torch.int16)), rep
            assert torch.count_nonzero(bufs[1]["ws"][:4 * B * Hkv]).item() == 0
            step(pools[0], bufs[0])            # eager work between replays
            torch.cuda.synchronize()
    finally:
        pba.set_validate(True)
    assert np.array_equal(to_bits(pools[1].k), opool.k) and np.array_equal(to_bits(pools[1].v), opool.v)
    ref, ref_lse = att.paged_decode(opool, qb, list(tables), lens, 1 / math.sqrt(D))
    assert np.max(np.abs(bufs[1]["out"].cpu().numpy() - ref)) <= TOL
    assert np.max(np.abs(bufs[1]["lse"].cpu().numpy() - ref_lse)) <= TOL
