"""Pins for oracle.layout: the pages' checked address trace and rejection order."""
import itertools

import numpy as np
import pytest

from oracle import layout
from oracle.layout import AddressRejected, CacheGroup, Descriptor


def _g1(fx):
    g = fx["checked_address"]["group"]
    d = fx["checked_address"]["descriptor_2001"]
    return CacheGroup(
        group_id=g["group_id"], layer_start=g["layer_start"], layer_end=g["layer_end"],
        block_size=g["block_size"], kv_heads_local=g["kv_heads_local"], head_dim=g["head_dim"],
        scalar_bytes=g["scalar_bytes"], shape=tuple(g["shape"]), axis_order=tuple(g["axis_order"]),
        base={"K": g["k_base"], "V": g["k_base"] + 2 ** 30}, pool_generation=g["pool_generation"],
        descriptors={2001: Descriptor(d["pool_generation"], d["physical_slot"], d["valid_rows"])})


def _g0():
    # layers [0, 24); only needed so layer 24 resolves to exactly one group.
    return CacheGroup(group_id=0, layer_start=0, layer_end=24, block_size=16, kv_heads_local=4,
                      head_dim=128, scalar_bytes=2, shape=(24, 8, 16, 4, 128),
                      axis_order=("layer_local", "physical_slot", "token_offset", "kv_head_local",
                                  "head_dim"),
                      base={"K": 0, "V": 2 ** 28})


def test_checked_address_trace(golden):
    fx = golden("address_trace.json")
    e = fx["checked_address"]["expect"]
    g1 = _g1(fx)
    assert layout.row_major_strides(g1.shape) == tuple(e["strides"])
    assert layout.element_offset(e["coordinate"], e["strides"]) == e["element_offset"]
    assert layout.token_to_block(16, 16) == (e["logical_block"], e["token_offset"])
    q = fx["checked_address"]["query"]
    tables = {0: [1000, 1001], 1: [2000, 2001]}
    sid, addr = layout.resolve_kv_address([_g0(), g1], 33, tables, q["token"], q["layer"],
                                          q["kind"], q["head"], q["lane"])
    assert sid == e["slot_id"] == 96
    assert addr == e["byte_address"] == 4_311_843_082
    assert addr - g1.base["K"] == e["byte_offset"]
    # A slot id is not a byte address.
    assert sid != addr


def test_visibility_dominates_shared_validity(golden):
    fx = golden("address_trace.json")
    v = fx["visibility"]
    g1 = _g1(fx)
    tables = {0: [1000, 1001], 1: [2000, 2001]}
    # Token 24 of a 25-token request is legal: logical block 1, offset 8.
    assert layout.token_to_block(v["legal"]["token"], 16) == (1, v["legal"]["offset"])
    layout.resolve_kv_address([_g0(), g1], v["context_length"], tables, 24, 24, "K", 0, 0)
    # Token 25 is rejected by visibility even though block 2001 holds 16 valid rows.
    with pytest.raises(AddressRejected) as exc:
        layout.resolve_kv_address([_g0(), g1], v["context_length"], tables, 25, 24, "K", 0, 0)
    assert exc.value.reason == "visibility"
    assert v["context_length"] - 16 == v["last_block_visible_rows"]


def test_rejection_order(golden):
    fx = golden("address_trace.json")
    g1 = _g1(fx)
    groups = [_g0(), g1]
    tables = {0: [1000], 1: [2000]}           # table too short for token 16
    with pytest.raises(AddressRejected) as exc:
        layout.resolve_kv_address(groups, 40, tables, 16, 24, "K", 0, 0)
    assert exc.value.reason == "table_bounds"
    tables = {0: [1000, 1001], 1: [2000, 2002]}  # 2002 has no descriptor
    with pytest.raises(AddressRejected) as exc:
        layout.resolve_kv_address(groups, 40, tables, 16, 24, "K", 0, 0)
    assert exc.value.reason == "identity"
    g1.descriptors[2003] = Descriptor(6, 3, 16)   # stale generation
    tables = {0: [1000, 1001], 1: [2000, 2003]}
    with pytest.raises(AddressRejected) as exc:
        layout.resolve_kv_address(groups, 40, tables, 16, 24, "K", 0, 0)
    assert exc.value.reason == "identity"
    g1.descriptors[2004] = Descriptor(7, 5, 2)    # only two committed rows
    tables = {0: [1000, 1001], 1: [2000, 2004]}
    layout.resolve_kv_address(groups, 40, tables, 17, 24, "K", 0, 0)
    with pytest.raises(AddressRejected) as exc:
        layout.resolve_kv_address(groups, 40, tables, 18, 24, "K", 0, 0)
    assert exc.value.reason == "validity"
    # Visibility is checked before everything else.
    with pytest.raises(AddressRejected) as exc:
        layout.resolve_kv_address(groups, 5, {0: [], 1: []}, 18, 24, "K", 0, 0)
    assert exc.value.reason == "visibility"


def test_boundary_crossing_slot_ids(golden):
    b = golden("address_trace.json")["boundary_crossing"]
    assert layout.token_to_block(b["token"], b["block_size"]) == (b["logical_block"], b["offset"])
    assert layout.slot_id(b["g0_physical_slot"], 16, b["offset"]) == b["g0_slot_id"] == 0
    assert layout.slot_id(b["g1_physical_slot"], 16, b["offset"]) == b["g1_slot_id"] == 64


def test_row_major_strides_match_numpy():
    # Independent check: numpy's C-order strides for the same shape.
    for shape in [(8, 8, 16, 4, 128), (3, 5, 7), (4096, 8, 64, 128), (1,)]:
        arr = np.empty(shape, dtype=np.uint8)
        assert layout.row_major_strides(shape) == arr.strides


def test_pool_element_offsets_match_numpy_indexing():
    nb, h, p, d = 5, 3, 16, 8
    for kind in ("K", "V"):
        shape = layout.pool_shape(kind, nb, h, p, d)
        flat = np.arange(int(np.prod(shape))).reshape(shape)
        for blk, head, tok, dim in itertools.product([0, 4], [0, 2], [0, 15], [0, 7]):
            idx = (blk, head, tok, dim) if kind == "K" else (blk, head, dim, tok)
            assert layout.pool_element_offset(kind, (nb, h, p, d), blk, head, tok, dim) == flat[idx]
