"""GPU parity of the cache-group calls (pba_kv_append_bundle,
pba_block_copy_bundle, pba_group_layer_pool) through the C ABI.

* Scripts over two groups (different block sizes, layer counts and memory
  orders) run on the oracle's bundle allocator; the bundle calls leave every
  group's K and V memory bit-identical to the oracle's layered pools, and to
  the same script issued as single-layer calls on every layer.
* Decode of every layer through the group's layer pool matches the oracle's
  binary64 decode of that layer (2e-3).
* Validate mode rejects half bundles, repeated and out-of-range slots and bad
  copy pairs before any group changes.
* The full 32-layer workload (the pages' two groups at one rank's share):
  decode of sampled layers against single-layer oracle pools.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from harness import (execute_bundle, gpu_bundle_groups, gpu_bundle_replay, oracle_bundle_pools,
                     to_bits, to_device)
from oracle import attention as att
from oracle.allocator import BlockAllocator  # noqa: F401  (documents the single-group twin)
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


def script(groups, dtype="bf16", d=128, H=2, Hq=8, seed_rep=0):
    w = wl.BundleWorkload("bundle", groups, Hq, H, d, dtype, wl.seed_for("bundle", seed_rep))
    w.actions = [("new",), ("prefill", 0, 150), ("new",), ("prefill", 1, 33), ("fork", 0),
                 ("fork", 1), ("append", 2), ("append", 3), ("append", 0), ("prefill", 2, 40),
                 ("release", 1), ("new",), ("prefill", 4, 70), ("fork", 4), ("append", 5),
                 ("prefill", 5, 17)]
    w.decode = [0, 2, 3, 4, 5]
    return w


CASES = [
    ("p16blk+p32lay", [wl.GroupShape(3, 16, 64, False), wl.GroupShape(2, 32, 40, True)], "bf16", 128),
    ("p64lay+p16blk", [wl.GroupShape(2, 64, 24, True), wl.GroupShape(4, 16, 64, False)], "bf16", 64),
    ("three groups", [wl.GroupShape(1, 16, 48, True), wl.GroupShape(2, 16, 48, False),
                      wl.GroupShape(3, 32, 32, True)], "bf16", 128),
    ("f32", [wl.GroupShape(2, 16, 64, False), wl.GroupShape(1, 32, 40, True)], "f32", 64),
]


def _gpu_rows(w, rows, dev):
    return [(to_device(k, w.dtype, dev), to_device(v, w.dtype, dev)) for k, v in rows]


@pytest.mark.parametrize("name,groups,dtype,d", CASES, ids=[c[0] for c in CASES])
def test_bundle_pools_bit_exact(pba, gpu, name, groups, dtype, d):
    w = script(groups, dtype, d)
    say("bundle pools", name, [(g.layers, g.block_size, g.num_blocks, g.layer_major) for g in groups])
    ex = execute_bundle(w)
    rows = [wl.bundle_rows(w, g) for g in range(len(groups))]
    pools = oracle_bundle_pools(ex, rows)
    rows_dev = _gpu_rows(w, rows, gpu)
    fused = gpu_bundle_groups(w, gpu)
    gpu_bundle_replay(ex, fused, rows_dev)
    split = gpu_bundle_groups(w, gpu)
    gpu_bundle_replay(ex, split, rows_dev, per_layer=True)
    torch.cuda.synchronize()
    for g, p in enumerate(pools):
        for kind, want in (("k", p.k), ("v", p.v)):
            got = to_bits(getattr(fused[g], kind)).reshape(-1)
            assert np.array_equal(got, want), (name, g, kind)
            assert np.array_equal(to_bits(getattr(split[g], kind)).reshape(-1), want)
    # Decode every layer of every group through its layer pool.
    B = len(w.decode)
    qall = wl.bundle_q_bits(w)
    scale = 1 / math.sqrt(d)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    layer = 0
    for g, grp in enumerate(fused):
        tab = torch.from_numpy(ex.tables[g]).to(gpu)
        for l in range(grp.num_layers):
            q = to_device(qall[layer], dtype, gpu)
            out, lse = pba.paged_decode(grp.layer(l), q, tab, lens, scale)
            torch.cuda.synchronize()
            ref, ref_lse = att.paged_decode(pools[g].layer_pool(l), qall[layer], list(ex.tables[g]),
                                            ex.seq_lens, scale)
            assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL, (name, g, l)
            assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= TOL
            layer += 1
    assert layer == w.total_layers and B == qall.shape[1]


def test_layer_pool_descriptor_matches_view(pba, gpu):
    w = script(CASES[0][1])
    groups = gpu_bundle_groups(w, gpu)
    for grp in groups:
        for l in range(grp.num_layers):
            a, b = grp.layer_desc(l), grp.layer(l).desc()
            assert all(getattr(a, f) == getattr(b, f) for f, _ in a._fields_)


def test_validate_rejections_leave_groups_unchanged(pba, gpu):
    w = script(CASES[0][1])
    ex = execute_bundle(w)
    groups = gpu_bundle_groups(w, gpu)
    rows = _gpu_rows(w, [wl.bundle_rows(w, g) for g in range(2)], gpu)
    gpu_bundle_replay(ex, groups, rows)
    torch.cuda.synchronize()
    before = [(g.k.clone(), g.v.clone()) for g in groups]
    say("bundle validate rejections")

    def slots(a, b):
        return [torch.tensor(a, dtype=torch.int64, device=gpu),
                torch.tensor(b, dtype=torch.int64, device=gpu)]

    k2 = [r[0][:2] for r in rows]
    v2 = [r[1][:2] for r in rows]
    cases = [
        (slots([5, 6], [7, -1]), -9),          # token 1 in group 0 only
        (slots([5, 6], [7, 7]), -7),           # repeated slot in group 1
        (slots([5, 64 * 16], [7, 8]), -6),     # beyond group 0's pool
    ]
    for sl, status in cases:
        with pytest.raises(pba.PBAError) as e:
            pba.kv_append_bundle(groups, sl, k2, v2)
        assert e.value.status == status
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=gpu)
    with pytest.raises(pba.PBAError) as e:            # group 1 pair overlaps itself
        pba.block_copy_bundle(groups, [i32([1]), i32([3])], [i32([2]), i32([3])])
    assert e.value.status == -7
    with pytest.raises(pba.PBAError) as e:
        pba.block_copy_bundle(groups, [i32([1]), i32([3])], [i32([2]), i32([40])])
    assert e.value.status == -6
    torch.cuda.synchronize()
    for g, (k, v) in zip(groups, before):
        assert torch.equal(g.k.view(torch.int16), k.view(torch.int16))
        assert torch.equal(g.v.view(torch.int16), v.view(torch.int16))
    # A token skipped in every group is fine; unequal copy counts are fine.
    pba.kv_append_bundle(groups, slots([-1, -1], [-1, -1]), k2, v2)
    pba.block_copy_bundle(groups, [i32([1]), i32([])], [i32([2]), i32([])])
    torch.cuda.synchronize()
    assert torch.equal(groups[1].k.view(torch.int16), before[1][0].view(torch.int16))


def test_layers32_sampled_layers(pba, gpu):
    """The 32-layer, two-group workload at full size: pools built by bundle
    calls; layers 0, 13, 23 (block-major group) and 24, 31 (layer-major
    group) decoded and checked on every row against single-layer oracle
    pools replayed with that layer's rows."""
    w = wl.layers32()
    ex = execute_bundle(w)
    say("layers32", [(g.layers, g.num_blocks) for g in w.groups], "writes", ex.n_writes,
        "batch", len(w.decode))
    rows = [wl.bundle_rows(w, g) for g in range(2)]
    groups = gpu_bundle_groups(w, gpu)
    gpu_bundle_replay(ex, groups, _gpu_rows(w, rows, gpu))
    torch.cuda.synchronize()
    qall = wl.bundle_q_bits(w)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    scale = 1 / math.sqrt(w.head_dim)
    sample = np.arange(len(w.decode))
    for model_layer in (0, 13, 23, 24, 31):
        g = 0 if model_layer < 24 else 1
        l = model_layer if g == 0 else model_layer - 24
        gs = w.groups[g]
        # Single-layer oracle pool of this layer (poisoned like the group's layer).
        nb, H, P, d = gs.num_blocks, w.num_kv_heads, gs.block_size, w.head_dim
        k0 = np.zeros((nb, H, P, d), dtype=np.uint16)
        v0 = np.zeros((nb, H, d, P), dtype=np.uint16)
        op = BitPool(k0, v0, "bf16")
        for o in ex.ops:
            if o[0] == "append":
                op.kv_append(o[1][g], rows[g][0][o[2]:o[3], l], rows[g][1][o[2]:o[3], l])
            elif o[1][g][0].size:
                op.block_copy(o[1][g][0], o[1][g][1])
        q = to_device(qall[model_layer], "bf16", gpu)
        tab = torch.from_numpy(ex.tables[g]).to(gpu)
        out, _ = pba.paged_decode(groups[g].layer(l), q, tab, lens, scale)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        ref, _ = att.paged_decode(op, qall[model_layer][sample], [ex.tables[g][i] for i in sample],
                                  ex.seq_lens[sample], scale)
        err = np.max(np.abs(out[sample] - ref))
        say("   layer", model_layer, "max err", err)
        assert err <= TOL
