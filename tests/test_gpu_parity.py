"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bars: kv_append, block_copy and the whole pool are bit exact; paged_decode is
within 2e-3 max-abs of the binary64 oracle (bf16 inputs, fp32 accumulation).
Every case prints its name, shapes and seed (flushed) before its GPU work.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from harness import execute, gpu_pool, gpu_replay, oracle_pool, to_bits, to_device
from oracle import attention as att
from oracle.pool import BitPool

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


def run_workload(pba, w, device, max_blocks=None, check_pool=True, pairs=None,
                 partition_tokens=0):
    say(w.name, w.shape, "seed", w.seed)
    ex = execute(w, max_blocks)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    pool = gpu_pool(ex, device)
    gpu_replay(ex, pool, to_device(k_rows, w.shape.dtype, device), to_device(v_rows, w.shape.dtype, device))
    torch.cuda.synchronize()
    if check_pool:
        assert np.array_equal(to_bits(pool.k), opool.k), "K pool bits differ"
        assert np.array_equal(to_bits(pool.v), opool.v), "V pool bits differ"
    qb = wl.q_bits(w)
    q = to_device(qb, w.shape.dtype, device)
    tables = torch.from_numpy(ex.tables).to(device)
    lens = torch.from_numpy(ex.seq_lens).to(device)
    scale = 1.0 / math.sqrt(w.shape.head_dim)
    out, lse = pba.paged_decode(pool, q, tables, lens, scale, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    ref_out, ref_lse = att.paged_decode(opool, qb, [t for t in ex.tables], ex.seq_lens, scale,
                                        rows=pairs)
    o = out.cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    sel = ~np.isnan(ref_out[..., 0])
    err = np.max(np.abs(o[sel] - ref_out[sel]))
    lerr = np.max(np.abs(l[sel] - ref_lse[sel]))
    say(w.name, "max abs err", err, "lse err", lerr)
    assert np.all(np.isfinite(o)), "non-finite output (a padding or stale row was read?)"
    assert err <= TOL
    assert lerr <= TOL
    return ex, pool, out, lse


def test_tiny(pba, gpu):
    ex, pool, out, lse = run_workload(pba, wl.tiny(), gpu)
    assert ex.alloc.table(0) == list(ex.tables[0]) and len(ex.tables[0]) == 3
    assert int(ex.seq_lens[0]) % 16 == 3


# ---------------------------------------------------------------------------
# Small random shapes: every supported P, d, G, dtype; ragged tails; splits.
# ---------------------------------------------------------------------------
SMALL = [
    # (dtype, P, d, Hkv, G, lengths)
    ("bf16", 16, 128, 2, 4, [1, 15, 16, 17, 33, 300]),
    ("bf16", 32, 128, 1, 8, [31, 32, 64, 65, 700]),
    ("bf16", 64, 64, 2, 1, [1, 63, 64, 129, 1000]),
    ("bf16", 128, 128, 3, 16, [5, 128, 257, 600]),
    ("bf16", 256, 64, 1, 2, [255, 256, 257, 1300]),
    ("f32", 16, 64, 1, 1, [35, 1, 16, 17]),
    ("f32", 64, 128, 2, 4, [3, 64, 65, 500]),
    ("f32", 256, 128, 1, 16, [256, 257, 900]),
]


def small_workload(dtype, P, d, Hkv, G, lengths, seed):
    nb = sum(-(-T // P) for T in lengths) + 7
    w = wl.Workload(f"small_{dtype}_P{P}_d{d}_G{G}", wl.Shape(P, Hkv * G, Hkv, d, dtype, nb), seed)
    for r, T in enumerate(lengths):
        w.actions.append(("new",))
        w.actions.append(("prefill", r, T))
    w.decode = list(range(len(lengths)))
    return w


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("partition_tokens", [0, 256, 512])
def test_small_shapes(pba, gpu, case, partition_tokens):
    dtype, P, d, Hkv, G, lengths = SMALL[case]
    w = small_workload(dtype, P, d, Hkv, G, lengths, 20261202 + 1000 + case)
    run_workload(pba, w, gpu, partition_tokens=partition_tokens)


def test_partition_count_and_placement_invariance(pba, gpu):
    """Bitwise-identical output under a permuted physical placement; close
    output across partition counts; deterministic reruns."""
    base = small_workload("bf16", 16, 128, 2, 4, [1, 40, 333, 1500, 2049], 20261202 + 2000)
    say("invariance", base.shape)
    ex = execute(base)
    k_rows, v_rows = wl.kv_rows(base, ex.n_writes)
    dev = gpu
    results = {}
    for variant in ("a", "b"):
        # A different free-FIFO order places the same logical rows elsewhere.
        w = small_workload("bf16", 16, 128, 2, 4, [1, 40, 333, 1500, 2049], 20261202 + 2000)
        if variant == "b":
            w.seed += 7  # changes only the FIFO order / poison (rows come from base)
        exv = execute(w)
        pool = gpu_pool(exv, dev)
        gpu_replay(exv, pool, to_device(k_rows, "bf16", dev), to_device(v_rows, "bf16", dev))
        q = to_device(wl.q_bits(base), "bf16", dev)
        tables = torch.from_numpy(exv.tables).to(dev)
        lens = torch.from_numpy(exv.seq_lens).to(dev)
        for pt in (256, 512, 2304):
            out, lse = pba.paged_decode(pool, q, tables, lens, partition_tokens=pt)
            out2, lse2 = pba.paged_decode(pool, q, tables, lens, partition_tokens=pt)
            torch.cuda.synchronize()
            assert torch.equal(out, out2) and torch.equal(lse, lse2), "non-deterministic"
            results[(variant, pt)] = (out.cpu(), lse.cpu())
        assert not np.array_equal(exv.tables, ex.tables) or variant == "a"
    for pt in (256, 512, 2304):
        assert torch.equal(results[("a", pt)][0], results[("b", pt)][0]), "placement changed bits"
    a256, a2304 = results[("a", 256)][0], results[("a", 2304)][0]
    assert (a256 - a2304).abs().max().item() <= 1e-4


def test_stream_ordered_copy_append_decode(pba, gpu):
    """copy -> append -> decode on a side stream with no host sync between."""
    w = wl.shared_prefix(children=4, prefix=40, lo=3, hi=9, num_blocks=64)
    say("stream order", w.shape)
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    pool = gpu_pool(ex, gpu)
    kd, vd = to_device(k_rows, "bf16", gpu), to_device(v_rows, "bf16", gpu)
    q = to_device(wl.q_bits(w), "bf16", gpu)
    tables = torch.from_numpy(ex.tables).to(gpu)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    torch.cuda.synchronize()
    pba.set_validate(False)
    try:
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            gpu_replay(ex, pool, kd, vd, stream=s)
            out, lse = pba.paged_decode(pool, q, tables, lens, stream=s)
        s.synchronize()
    finally:
        pba.set_validate(True)
    assert np.array_equal(to_bits(pool.k), opool.k) and np.array_equal(to_bits(pool.v), opool.v)
    ref, _ = att.paged_decode(opool, wl.q_bits(w), list(ex.tables), ex.seq_lens,
                              1 / math.sqrt(128))
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL


def test_negative_slots_and_empty_calls(pba, gpu):
    say("negative slots")
    pool = pba.KVPool.empty(4, 16, 2, 64, torch.bfloat16, gpu)
    pool.k.view(torch.int16).fill_(0x7FC1)
    pool.v.view(torch.int16).fill_(0x7FC1)
    before_k, before_v = to_bits(pool.k).copy(), to_bits(pool.v).copy()
    rows = torch.randn(3, 2, 64, device=gpu).to(torch.bfloat16)
    slots = torch.tensor([-1, 5, -7], dtype=torch.int64, device=gpu)
    pba.kv_append(pool, slots, rows, rows)
    torch.cuda.synchronize()
    k, v = to_bits(pool.k), to_bits(pool.v)
    rb = to_bits(rows)
    assert np.array_equal(k[0, :, 5, :], rb[1]) and np.array_equal(v[0, :, :, 5], rb[1])
    k[0, :, 5, :] = before_k[0, :, 5, :]
    v[0, :, :, 5] = before_v[0, :, :, 5]
    assert np.array_equal(k, before_k) and np.array_equal(v, before_v)
    empty64 = torch.empty(0, dtype=torch.int64, device=gpu)
    empty32 = torch.empty(0, dtype=torch.int32, device=gpu)
    pba.kv_append(pool, empty64, rows[:0], rows[:0])
    pba.block_copy(pool, empty32, empty32)
    out, lse = pba.paged_decode(pool, torch.empty(0, 4, 64, dtype=torch.bfloat16, device=gpu),
                                torch.empty(0, 2, dtype=torch.int32, device=gpu), empty32)
    assert out.shape == (0, 4, 64)


def test_validate_mode_rejects_and_preserves_pool(pba, gpu):
    say("validate mode")
    pool = pba.KVPool.empty(4, 16, 1, 64, torch.bfloat16, gpu)
    pool.k.view(torch.int16).fill_(0x1234)
    pool.v.view(torch.int16).fill_(0x4321)
    before = (to_bits(pool.k).copy(), to_bits(pool.v).copy())
    rows = torch.randn(2, 1, 64, device=gpu).to(torch.bfloat16)
    i64 = lambda x: torch.tensor(x, dtype=torch.int64, device=gpu)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=gpu)
    with pytest.raises(pba.PBAError) as e:
        pba.kv_append(pool, i64([3, 64]), rows, rows)          # slot 64 = 4 blocks * 16
    assert e.value.status == -6
    with pytest.raises(pba.PBAError) as e:
        pba.kv_append(pool, i64([3, 3]), rows, rows)
    assert e.value.status == -7
    with pytest.raises(pba.PBAError) as e:
        pba.block_copy(pool, i32([0, 1]), i32([2, 2]))
    assert e.value.status == -7
    with pytest.raises(pba.PBAError) as e:
        pba.block_copy(pool, i32([0, 1]), i32([1, 3]))
    assert e.value.status == -7
    with pytest.raises(pba.PBAError) as e:
        pba.block_copy(pool, i32([4]), i32([1]))
    assert e.value.status == -6
    q = torch.randn(1, 1, 64, device=gpu).to(torch.bfloat16)
    for tab, T in [([0, 9], 20), ([0, 1], 33), ([0, 1], 0), ([-1, 1], 5)]:
        with pytest.raises(pba.PBAError) as e:
            pba.paged_decode(pool, q, i32([tab]), i32([T]))
        assert e.value.status == -6
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(pool.k), before[0]) and np.array_equal(to_bits(pool.v), before[1])
    # Entries past ceil(T/P) are never read: -1 padding is fine.
    out, _ = pba.paged_decode(pool, q, i32([[2, -1]]), i32([16]))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_block_copy_bit_exact_nan_payloads(pba, gpu):
    say("block copy NaN payloads")
    k0, v0 = wl.pool_poison(wl.Workload("x", wl.Shape(64, 4, 4, 128, "bf16", 12), 99))
    pool = pba.KVPool(to_device(k0, "bf16", gpu), to_device(v0, "bf16", gpu))
    src = np.array([3, 0, 11, 5], dtype=np.int32)
    dst = np.array([7, 1, 2, 9], dtype=np.int32)
    opool = BitPool(k0, v0, "bf16")
    opool.block_copy(src, dst)
    pba.block_copy(pool, torch.from_numpy(src).to(gpu), torch.from_numpy(dst).to(gpu))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(pool.k), opool.k) and np.array_equal(to_bits(pool.v), opool.v)


def test_workspace_counters_reset_between_calls(pba, gpu):
    """One zeroed workspace, calls with different partition counts per row:
    every call must leave the completion counters at zero for the next."""
    base = small_workload("bf16", 64, 128, 2, 8, [3000, 700, 2048, 1], 20261202 + 4000)
    say("workspace reuse", base.shape)
    ex = execute(base)
    k_rows, v_rows = wl.kv_rows(base, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    pool = gpu_pool(ex, gpu)
    gpu_replay(ex, pool, to_device(k_rows, "bf16", gpu), to_device(v_rows, "bf16", gpu))
    qb = wl.q_bits(base)
    q = to_device(qb, "bf16", gpu)
    tables = torch.from_numpy(ex.tables).to(gpu)
    B, Hq = qb.shape[0], qb.shape[1]
    ws_bytes = pba.paged_decode_workspace_bytes(pool, Hq, B, ex.tables.shape[1], 256)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=gpu)
    scale = 1 / math.sqrt(128)
    outs = []
    for lens in ([3000, 700, 2048, 1], [257, 650, 1024, 1], [3000, 700, 2048, 1], [1, 1, 1, 1],
                 [3000, 700, 2048, 1]):
        ld = torch.tensor(lens, dtype=torch.int32, device=gpu)
        out, lse = pba.paged_decode(pool, q, tables, ld, scale, partition_tokens=256, workspace=ws)
        torch.cuda.synchronize()
        ref, _ = att.paged_decode(opool, qb, list(ex.tables), lens, scale)
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL, lens
        outs.append(out.clone())
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[0], outs[4])
    n_counters = B * base.shape.num_kv_heads
    assert torch.count_nonzero(ws[:4 * n_counters]).item() == 0


def test_graph_replay_matches_eager(pba, gpu):
    """The decode step (block_copy -> kv_append -> paged_decode with a split
    and its fused merge) captured in a HIP graph.  Every replay, with eager
    library calls and synchronisations between replays, must equal the eager
    step bit for bit (pool bytes, out, lse), and the oracle within TOL.  No
    call of the step records a memset: the workspace counters return to zero
    inside the kernel."""
    import bench

    w = wl.shared_prefix(children=6, prefix=300, lo=3, hi=40, num_blocks=160)
    say("graph replay", w.shape, "seed", w.seed)
    plan = bench.plan_script(w)
    assert len(plan.step_src) > 0 and len(plan.step_slots) == 6
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    dt = w.shape.dtype
    kd, vd = to_device(k_rows, dt, gpu), to_device(v_rows, dt, gpu)
    k0, v0 = wl.pool_poison(w)
    pools = [pba.KVPool(to_device(k0, dt, gpu), to_device(v0, dt, gpu)) for _ in range(2)]
    for pool in pools:
        for op in plan.setup:
            if op[0] == "copy":
                pba.block_copy(pool, torch.from_numpy(op[1]).to(gpu), torch.from_numpy(op[2]).to(gpu))
            else:
                pba.kv_append(pool, torch.from_numpy(op[1]).to(gpu), kd[op[2]:op[3]], vd[op[2]:op[3]])
    lo, hi = plan.step_rows
    slots = torch.from_numpy(plan.step_slots).to(gpu)
    src = torch.from_numpy(plan.step_src).to(gpu)
    dst = torch.from_numpy(plan.step_dst).to(gpu)
    q = to_device(wl.q_bits(w), dt, gpu)
    tables = torch.from_numpy(plan.tables).to(gpu)
    lens = torch.from_numpy(plan.seq_lens).to(gpu)
    B, Hq, D = q.shape
    pt = 256
    ws_bytes = pba.paged_decode_workspace_bytes(pools[0], Hq, B, plan.tables.shape[1], pt)
    assert ws_bytes > 0
    bufs = [dict(out=torch.empty((B, Hq, D), dtype=torch.float32, device=gpu),
                 lse=torch.empty((B, Hq), dtype=torch.float32, device=gpu),
                 ws=torch.zeros(ws_bytes, dtype=torch.uint8, device=gpu)) for _ in range(2)]

    def step(pool, b):
        pba.block_copy(pool, src, dst)
        pba.kv_append(pool, slots, kd[lo:hi], vd[lo:hi])
        pba.paged_decode(pool, q, tables, lens, out=b["out"], lse=b["lse"], partition_tokens=pt,
                         workspace=b["ws"])

    pba.set_validate(False)
    try:
        step(pools[0], bufs[0])                    # eager reference
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(pools[1], bufs[1])                # warm the graph's buffers once
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
            assert torch.count_nonzero(bufs[1]["ws"][:4 * B * w.shape.num_kv_heads]).item() == 0
            step(pools[0], bufs[0])                # eager work between replays
            torch.cuda.synchronize()
    finally:
        pba.set_validate(True)
    assert np.array_equal(to_bits(pools[1].k), opool.k) and np.array_equal(to_bits(pools[1].v), opool.v)
    ref, ref_lse = att.paged_decode(opool, wl.q_bits(w), list(ex.tables), ex.seq_lens,
                                    1 / math.sqrt(D))
    assert np.max(np.abs(bufs[1]["out"].cpu().numpy() - ref)) <= TOL
