"""Host-only checks of the cache-group ABI (no kernel runs): layer
descriptors, the tile-disjointness rule, and rejections of bad group
descriptors and bundle arguments before any launch."""
import ctypes

import pytest
import torch

NULL = None


def _pba():
    import block_table_attention_amd as pba
    return pba


def _group(layer_major=True, L=3, NB=10, H=2, P=16, d=128, dtype=torch.bfloat16):
    pba = _pba()
    return pba.KVGroup.empty(L, NB, P, H, d, dtype=dtype, device="cpu", layer_major=layer_major)


@pytest.mark.parametrize("layer_major", [True, False])
def test_layer_descriptors(layer_major):
    """pba_group_layer_pool gives the same descriptor as the torch view of the
    layer, and its K/V element addresses follow the group's stride rule."""
    g = _group(layer_major)
    es = 2
    for layer in range(g.num_layers):
        mine = g.layer_desc(layer)
        view = g.layer(layer).desc()
        for f, _ in mine._fields_:
            assert getattr(mine, f) == getattr(view, f), (layer, f)
        # Element (layer, block 7, head 1, token 3, dim 5) of K, and its V twin.
        b, h, o, c = 7, 1, 3, 5
        k_addr = mine.k + es * (b * mine.k_stride_block + h * mine.k_stride_head + o * 128 + c)
        v_addr = mine.v + es * (b * mine.v_stride_block + h * mine.v_stride_head + c * 16 + o)
        kt = g.k[layer, b] if layer_major else g.k[b, layer]
        vt = g.v[layer, b] if layer_major else g.v[b, layer]
        assert k_addr == kt[h, o, c].data_ptr() and v_addr == vt[h, c, o].data_ptr()


def test_layer_index_rejected():
    pba = _pba()
    g = _group()
    out = pba.PoolDesc()
    lib = pba._lib
    assert lib.pba_group_layer_pool(ctypes.byref(g.desc()), 3, ctypes.byref(out)) == -3
    assert lib.pba_group_layer_pool(ctypes.byref(g.desc()), -1, ctypes.byref(out)) == -3
    assert lib.pba_group_layer_pool(ctypes.byref(g.desc()), 0, NULL) == -1
    assert lib.pba_group_layer_pool(NULL, 0, ctypes.byref(out)) == -1


def _desc_with(g, **kw):
    pba = _pba()
    d = g.desc()
    new = pba.GroupDesc()
    ctypes.pointer(new)[0] = d
    for k, v in kw.items():
        if k.startswith("pool_"):
            setattr(new.pool, k[5:], v)
        else:
            setattr(new, k, v)
    return new


@pytest.mark.parametrize("layer_major,kw,status", [
    (True, dict(num_layers=0), -3),
    (True, dict(reserved0=1), -3),
    (True, dict(pool_split_log2=1), -4),
    (True, dict(k_stride_layer=-2048), -3),
    (True, dict(k_stride_layer=2048 * 2 * 10 - 2048), -3),  # layer 1 overlaps layer 0's last block
    (True, dict(v_stride_layer=4), -4),                    # not a multiple of 16 bytes
    (False, dict(k_stride_layer=2048), -3),                # layers overlap the heads
    (False, dict(pool_k_stride_block=2048 * 2 * 3 - 2048), -3),
    (True, dict(pool_k_stride_head=1024), -3),
])
def test_group_rejections(layer_major, kw, status):
    pba = _pba()
    g = _group(layer_major)
    bad = _desc_with(g, **kw)
    lib = pba._lib
    out = pba.PoolDesc()
    assert lib.pba_group_layer_pool(ctypes.byref(bad), 0, ctypes.byref(out)) == status
    arr = (pba.GroupDesc * 1)(bad)
    one = (ctypes.c_void_p * 1)(0x10000)
    assert lib.pba_kv_append_bundle(arr, 1, one, one, one, 4, NULL) == status
    cnt = (ctypes.c_int64 * 1)(2)
    assert lib.pba_block_copy_bundle(arr, 1, one, one, cnt, NULL) == status


def test_pool_overlap_rule():
    """A single-layer pool whose block stride is one tile while two heads
    share it would alias block b+1 head 0 with block b head 1."""
    pba = _pba()
    d = pba.PoolDesc(0x10000, 0x20000, 1, 8, 16, 2, 128, 0, 2048, 2048, 2 * 2048, 2048)
    assert pba._lib.pba_kv_append(ctypes.byref(d), 0x30000, 1, 0x40000, 0x50000, NULL) == -3
    # Head-major pools (heads outermost) are disjoint and accepted.
    hm = pba.PoolDesc(0x10000, 0x20000, 1, 8, 16, 2, 128, 0, 2048, 8 * 2048, 2048, 8 * 2048)
    assert pba._lib.pba_kv_append(ctypes.byref(hm), NULL, 0, NULL, NULL, NULL) == 0


def test_bundle_argument_rejections():
    pba = _pba()
    lib = pba._lib
    g = _group()
    arr = (pba.GroupDesc * 2)(g.desc(), g.desc())
    ptrs = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    nulls = (ctypes.c_void_p * 2)(0x10000, None)
    cnt = (ctypes.c_int64 * 2)(1, 1)
    assert lib.pba_kv_append_bundle(arr, 0, ptrs, ptrs, ptrs, 4, NULL) == -3
    assert lib.pba_kv_append_bundle(arr, 9, ptrs, ptrs, ptrs, 4, NULL) == -4
    assert lib.pba_kv_append_bundle(NULL, 1, ptrs, ptrs, ptrs, 4, NULL) == -1
    assert lib.pba_kv_append_bundle(arr, 2, ptrs, ptrs, ptrs, -1, NULL) == -3
    assert lib.pba_kv_append_bundle(arr, 2, nulls, ptrs, ptrs, 4, NULL) == -1
    assert lib.pba_kv_append_bundle(arr, 2, ptrs, ptrs, (ctypes.c_void_p * 2)(0x10008, 0x20000),
                                    4, NULL) == -4
    assert lib.pba_kv_append_bundle(arr, 2, NULL, NULL, NULL, 0, NULL) == 0
    assert lib.pba_block_copy_bundle(arr, 2, nulls, ptrs, cnt, NULL) == -1
    assert lib.pba_block_copy_bundle(arr, 2, ptrs, ptrs, (ctypes.c_int64 * 2)(1, -1), NULL) == -3
    assert lib.pba_block_copy_bundle(arr, 2, ptrs, ptrs, NULL, NULL) == -1
    assert lib.pba_block_copy_bundle(arr, 2, nulls, nulls, (ctypes.c_int64 * 2)(0, 0), NULL) == 0


def test_binding_shape_checks():
    pba = _pba()
    g = _group()
    slots = torch.zeros(4, dtype=torch.int64)
    rows = torch.zeros(4, 3, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pba.kv_append_bundle([g], [slots], [rows[:, :2].contiguous()], [rows])
    with pytest.raises(ValueError):
        pba.kv_append_bundle([g, g], [slots], [rows], [rows])
    with pytest.raises(ValueError):
        pba.block_copy_bundle([g], [torch.zeros(2, dtype=torch.int32)],
                              [torch.zeros(3, dtype=torch.int32)])
    with pytest.raises(ValueError):
        pba.KVGroup(g.k, g.v[:, :, :, :, :8])


def test_bench_bundle_plan_matches_oracle():
    """bench.py's multi-group plan (package BundleManager) equals the oracle
    bundle allocator's trace on the 32-layer workload's script: tables,
    lengths, and the multiset of every group's copies and writes."""
    import numpy as np

    import bench
    import workloads as wl
    from harness import execute_bundle

    w = wl.layers32(batch=12, forks=4)
    plan = bench.plan_bundle_script(w)
    ex = execute_bundle(w)
    for g in range(2):
        assert np.array_equal(plan.tables[g], ex.tables[g])
    assert np.array_equal(plan.seq_lens, ex.seq_lens)
    assert plan.n_writes == ex.n_writes
    for g in range(2):
        mine, theirs = [], []
        for op in plan.setup:
            if op[0] == "copy":
                mine += [("copy", int(s), int(d)) for s, d in zip(*op[1][g])]
            else:
                mine += [("write", int(s), r) for s, r in zip(op[1][g], range(op[2], op[3]))]
        lo, hi = plan.step_rows
        mine += [("copy", int(s), int(d)) for s, d in zip(*plan.step_copies[g])]
        mine += [("write", int(s), r) for s, r in zip(plan.step_slots[g], range(lo, hi))]
        for op in ex.ops:
            if op[0] == "copy":
                theirs += [("copy", int(s), int(d)) for s, d in zip(*op[1][g])]
            else:
                theirs += [("write", int(s), r) for s, r in zip(op[1][g], range(op[2], op[3]))]
        assert sorted(mine) == sorted(theirs)
    # Every forked pair copies its shared tail in both groups during the step.
    n_fork_tails = sum(1 for T in ex.seq_lens[:4] if (int(T) - 1) % 16)
    assert [len(c[0]) for c in plan.step_copies] == [n_fork_tails] * 2


# ---------------------------------------------------------------------------
# Contiguous arenas and the slot-indexed decode: host-side rejections
# ---------------------------------------------------------------------------
def _vkv_cfg(**kw):
    pba = _pba()
    d = dict(dtype=1, num_layers=2, num_slots=4, num_kv_heads=2, head_dim=128, block_size=16,
             max_tokens=300, page_bytes=65536, num_handles=0)
    d.update(kw)
    return pba.VkvConfig(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), -2),
    (dict(num_layers=0), -3),
    (dict(num_slots=0), -3),
    (dict(max_tokens=0), -3),
    (dict(page_bytes=0), -3),
    (dict(num_handles=-4), -3),
    (dict(head_dim=96), -4),
    (dict(block_size=8), -4),
    (dict(block_size=48), -4),
])
def test_arena_config_rejections(kw, status):
    """Rejected before any HIP call (these run without a GPU)."""
    pba = _pba()
    h = ctypes.c_void_p()
    assert pba._lib.pba_vkv_create(ctypes.byref(_vkv_cfg(**kw)), ctypes.byref(h)) == status
    assert not h.value
    assert pba._lib.pba_vkv_create(NULL, ctypes.byref(h)) == -1
    assert pba._lib.pba_vkv_map(NULL, 0, 1) == -1
    assert pba._lib.pba_vkv_free(NULL, 0, 1) == -1
    assert pba._lib.pba_vkv_destroy(NULL) == -1


def test_contiguous_decode_host_rejections():
    pba = _pba()
    lib = pba._lib
    d = pba.PoolDesc(0x10000, 0x20000, 1, 64, 16, 2, 128, 0, 2 * 16 * 128, 16 * 128,
                     2 * 16 * 128, 16 * 128)
    call = lambda desc, bps: lib.pba_paged_decode_contiguous(
        ctypes.byref(desc), 0x30000, 8, 0x40000, bps, 0x50000, 2, ctypes.c_float(0.1), 0x60000,
        NULL, 0, NULL, 0, NULL)
    assert call(d, 5) == -3                    # 64 blocks are not whole slots of 5
    assert call(d, 0) == -3
    f32 = pba.PoolDesc(0x10000, 0x20000, 0, 64, 16, 2, 128, 0, 2 * 16 * 128, 16 * 128,
                       2 * 16 * 128, 16 * 128)
    assert call(f32, 8) == -4                  # bf16 only
    split = pba.PoolDesc(0x10000, 0x20000, 1, 64, 16, 2, 128, 1, 2 * 32 * 128, 32 * 128,
                         2 * 32 * 128, 32 * 128)
    assert call(split, 8) == -4
    assert lib.pba_paged_decode_contiguous(ctypes.byref(d), NULL, 8, NULL, 8, NULL, 0,
                                           ctypes.c_float(0.1), NULL, NULL, 0, NULL, 0, NULL) == 0
