"""Token position -> block table entry -> slot id -> byte address.

Test infrastructure only (see ``oracle/__init__.py``).

Follows "M5.3 - KV Memory Layout and Exact Reuse":
  * section 0x03C: j = floor(t / P), o = t mod P, p = table[j], plus the four
    legality checks (request visibility, table bounds, physical identity,
    physical validity);
  * section 0x03D: slot id = physical_slot * P + o (a slot id is not an address);
  * section 0x03E: stride[a] = product of the dimensions right of axis a,
    element offset = sum(coordinate[a] * stride[a]), byte offset = scalar bytes
    * element offset, byte address = base[K or V] + byte offset;
  * section 0x03G: visibility is checked before physical validity, so a request
    never reads rows a longer request materialised in a shared block;
  * section 0x03I: the rejection order of the checked translator.

The library's pool layout is expressed with the same stride rule:
K is [num_blocks, H_kv, P, d] (axes block, head, token, dim) and V is
[num_blocks, H_kv, d, P] (axes block, head, dim, token).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Mapping, Sequence, Tuple


class AddressRejected(ValueError):
    """A read that the checked translator refuses; ``reason`` names the check."""

    def __init__(self, reason: str, detail: str = ""):
        super().__init__(f"{reason}: {detail}" if detail else reason)
        self.reason = reason


def row_major_strides(shape: Sequence[int]) -> Tuple[int, ...]:
    """stride[a] = prod(shape[b] for b > a)   (section 0x03E)."""
    strides = []
    acc = 1
    for dim in reversed(shape):
        strides.append(acc)
        acc *= int(dim)
    return tuple(reversed(strides))


def element_offset(coordinate: Sequence[int], strides: Sequence[int]) -> int:
    """E = sum_a I_a * S_a   (section 0x03E)."""
    if len(coordinate) != len(strides):
        raise ValueError("coordinate rank differs from stride rank")
    return sum(int(i) * int(s) for i, s in zip(coordinate, strides))


def token_to_block(token: int, block_size: int) -> Tuple[int, int]:
    """(logical block j, in-block offset o) = (floor(t/P), t mod P)  (0x03C)."""
    return token // block_size, token % block_size


def slot_id(physical_slot: int, block_size: int, offset: int) -> int:
    """slot = physical_slot * P + o   (section 0x03D)."""
    return physical_slot * block_size + offset


@dataclass(frozen=True)
class Descriptor:
    """What a physical block id resolves to in its pool generation (0x03F)."""

    pool_generation: int
    physical_slot: int
    valid_rows: int


@dataclass
class CacheGroup:
    """One cache group's layout manifest (sections 0x03B, 0x03E, 0x03I)."""

    group_id: int
    layer_start: int
    layer_end: int  # exclusive
    block_size: int
    kv_heads_local: int
    head_dim: int
    scalar_bytes: int
    shape: Tuple[int, ...]
    axis_order: Tuple[str, ...]
    base: Mapping[str, int]
    pool_generation: int = 0
    descriptors: Dict[int, Descriptor] = field(default_factory=dict)

    def end(self, kind: str) -> int:
        size = 1
        for d in self.shape:
            size *= d
        return self.base[kind] + self.scalar_bytes * size


def _unique_group(groups: Sequence[CacheGroup], layer: int) -> CacheGroup:
    hits = [g for g in groups if g.layer_start <= layer < g.layer_end]
    if len(hits) != 1:
        raise AddressRejected("layer_group", f"layer {layer} maps to {len(hits)} groups")
    return hits[0]


def resolve_kv_address(
    groups: Sequence[CacheGroup],
    context_length: int,
    tables_by_group: Mapping[int, Sequence[int]],
    token: int,
    layer: int,
    kind: str,
    head: int,
    lane: int,
) -> Tuple[int, int]:
    """Checked translator of section 0x03I; returns (slot_id, byte_address).

    Rejection order: request visibility, layer group, table bounds, physical
    identity (descriptor in the current pool generation), physical validity
    (offset < valid rows), head and lane bounds, tensor extent.
    """
    if not 0 <= token < context_length:
        raise AddressRejected("visibility", f"token {token} outside context {context_length}")
    group = _unique_group(groups, layer)
    layer_local = layer - group.layer_start
    logical_block, offset = token_to_block(token, group.block_size)
    table = tables_by_group[group.group_id]
    if not logical_block < len(table):
        raise AddressRejected("table_bounds", f"logical block {logical_block} >= {len(table)}")
    physical_id = table[logical_block]
    desc = group.descriptors.get(physical_id)
    if desc is None or desc.pool_generation != group.pool_generation:
        raise AddressRejected("identity", f"block {physical_id} unknown or stale")
    if not offset < desc.valid_rows:
        raise AddressRejected("validity", f"offset {offset} >= valid rows {desc.valid_rows}")
    if not 0 <= head < group.kv_heads_local:
        raise AddressRejected("head", f"head {head}")
    if not 0 <= lane < group.head_dim:
        raise AddressRejected("lane", f"lane {lane}")

    sid = slot_id(desc.physical_slot, group.block_size, offset)
    coordinate = {
        "layer_local": layer_local,
        "physical_slot": desc.physical_slot,
        "token_offset": offset,
        "kv_head_local": head,
        "head_dim": lane,
    }
    ordered = [coordinate[a] for a in group.axis_order]
    e = element_offset(ordered, row_major_strides(group.shape))
    address = group.base[kind] + group.scalar_bytes * e
    if not group.base[kind] <= address < group.end(kind):
        raise AddressRejected("extent", f"address {address} outside tensor")
    return sid, address


# ---------------------------------------------------------------------------
# The library's pool layout, written with the same stride rule.
# ---------------------------------------------------------------------------
K_AXES = ("block", "head", "token", "dim")
V_AXES = ("block", "head", "dim", "token")


def pool_shape(kind: str, num_blocks: int, kv_heads: int, block_size: int, head_dim: int):
    if kind == "K":
        return (num_blocks, kv_heads, block_size, head_dim)
    if kind == "V":
        return (num_blocks, kv_heads, head_dim, block_size)
    raise ValueError(kind)


def pool_element_offset(kind: str, shape_args: Tuple[int, int, int, int],
                        block: int, head: int, token_offset: int, dim: int) -> int:
    """Element offset of (block, head, in-block token, dim) in a K or V pool."""
    shape = pool_shape(kind, *shape_args)
    axes = K_AXES if kind == "K" else V_AXES
    coord = {"block": block, "head": head, "token": token_offset, "dim": dim}
    return element_offset([coord[a] for a in axes], row_major_strides(shape))
