"""Paged block-table attention for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libpba.so`` (declared in ``include/pba.h``).  The
functions below only marshal torch tensors into the C ABI: every step of
kv_append, block_copy and paged_decode runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from collections import OrderedDict
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

__all__ = ["KVPool", "kv_append", "block_copy", "paged_decode", "paged_decode_plan",
           "paged_decode_noalloc", "paged_decode_append", "paged_decode_plan_ex",
           "shared_plan_build", "PARTITIONS_AUTO",
           "paged_decode_ragged", "expand_block_tables", "pack_block_tables",
           "paged_decode_shared", "paged_decode_shared_workspace_bytes", "SharedPlan",
           "paged_decode_workspace_bytes", "decode_workspace", "KVGroup", "kv_append_bundle",
           "block_copy_bundle", "VKVArena", "paged_decode_contiguous", "set_validate", "PBAError",
           "lib_path", "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """The in-tree library, or the file named by PBA_LIB (a build kept elsewhere)."""
    return os.environ.get("PBA_LIB") or os.path.join(_HERE, "libpba.so")


if not os.path.exists(lib_path()):
    raise ImportError(
        f"{lib_path()} is missing: build it with `python block_table_attention_amd/build.py` "
        "(or __graft_entry__.build()); there is no fallback path")

_lib = ctypes.CDLL(lib_path())

PBA_F32, PBA_BF16 = 0, 1
STATUS = {0: "PBA_OK", -1: "PBA_ERR_NULL_ARG", -2: "PBA_ERR_BAD_DTYPE", -3: "PBA_ERR_BAD_SHAPE",
          -4: "PBA_ERR_UNSUPPORTED", -5: "PBA_ERR_WORKSPACE_TOO_SMALL",
          -6: "PBA_ERR_OUT_OF_RANGE", -7: "PBA_ERR_OVERLAP", -8: "PBA_ERR_HIP",
          -9: "PBA_ERR_HALF_BUNDLE", -10: "PBA_ERR_OUT_OF_MEMORY", -11: "PBA_ERR_SCRATCH_LIMIT"}
NOALLOC_COUNTER_BYTES = 256 * 1024        # PBA_NOALLOC_COUNTER_BYTES
NOALLOC_STATE_BYTES = 32 * 1024 * 1024    # PBA_NOALLOC_STATE_BYTES
MAX_GROUPS = 8
PARTITIONS_BALANCED = -1   # partition_tokens: balance the batch's chunks over the CUs
PARTITIONS_AUTO = -2       # paged_decode_plan_ex: the library chooses from the lengths
PLAN_REASONS = {0: "none", 1: "requested", 2: "table width", 3: "uniform lengths",
                4: "few rows", 5: "ragged lengths", 6: "mildly ragged lengths",
                7: "fallback: fp32 pool", 8: "fallback: more than 2048 rows",
                9: "fallback: LDS above 64 KiB", 10: "fallback: chunk count"}
DECOMPOSITIONS = {0: "grid", 1: "balanced"}
_DTYPES = {torch.float32: PBA_F32, torch.bfloat16: PBA_BF16}


class PoolDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("split_log2", ctypes.c_int32), ("k_stride_block", ctypes.c_int64),
                ("k_stride_head", ctypes.c_int64), ("v_stride_block", ctypes.c_int64),
                ("v_stride_head", ctypes.c_int64)]


class GroupDesc(ctypes.Structure):
    _fields_ = [("pool", PoolDesc), ("num_layers", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("k_stride_layer", ctypes.c_int64), ("v_stride_layer", ctypes.c_int64)]


class VkvConfig(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("page_bytes", ctypes.c_int64),
                ("num_handles", ctypes.c_int64)]


class VkvLedgers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "reserved_bytes", "pool_bytes", "mapped_bytes", "inactive_retained_bytes", "free_bytes",
        "bundle_maps", "bundle_unmaps", "slot_bytes")]


class SharedPlanDesc(ctypes.Structure):
    _fields_ = [("num_items", ctypes.c_int32), ("max_slots", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("private_parts", ctypes.c_int32),
                ("items", ctypes.c_void_p), ("row_private", ctypes.c_void_p),
                ("private_tokens", ctypes.c_int32), ("reserved0", ctypes.c_int32)]


class LengthHint(ctypes.Structure):
    _fields_ = [("sum_tokens", ctypes.c_int64), ("max_tokens", ctypes.c_int32),
                ("reserved0", ctypes.c_int32)]


class DecodePlanInfo(ctypes.Structure):
    _fields_ = [("partition_request", ctypes.c_int32), ("decomposition", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("num_partitions", ctypes.c_int32),
                ("reason", ctypes.c_int32), ("fallback", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


class SharedPlanParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "block_size", "group", "partition_tokens", "threshold", "tiles_per_item", "reserved0")]


class SharedPlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_items", "num_chunks", "max_slots", "private_parts", "private_tokens",
        "partition_tokens")] + [(n, ctypes.c_int64) for n in (
            "chunk_rows", "kv_rows_read", "chunk_visits", "partial_states")]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_P = ctypes.POINTER(PoolDesc)
_SP = ctypes.POINTER(SharedPlanDesc)
_GP = ctypes.POINTER(GroupDesc)
_SIGS = {
    "pba_kv_append": (ctypes.c_int, [_P, _vp, _i64, _vp, _vp, _vp]),
    "pba_block_copy": (ctypes.c_int, [_P, _vp, _vp, _i64, _vp]),
    "pba_paged_decode": (ctypes.c_int, [_P, _vp, _i32, _vp, _i32, _vp, _i32, ctypes.c_float, _vp,
                                        _vp, _i32, _vp, _sz, _vp]),
    "pba_paged_decode_append": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _i32,
                                               ctypes.c_float, _vp, _vp, _i32, _vp, _sz, _vp]),
    "pba_paged_decode_workspace_bytes": (_sz, [_P, _i32, _i32, _i32, _i32]),
    "pba_paged_decode_plan_ex": (ctypes.c_int, [_P, _i32, _i32, _i32, _i32,
                                                ctypes.POINTER(LengthHint),
                                                ctypes.POINTER(DecodePlanInfo)]),
    "pba_shared_plan_build": (ctypes.c_int, [_vp, _i32, _vp, _i32, ctypes.POINTER(SharedPlanParams),
                                             _vp, _vp, _i32, _vp, _vp, _i32,
                                             ctypes.POINTER(SharedPlanInfo)]),
    "pba_paged_decode_plan": (ctypes.c_int, [_P, _i32, _i32, _i32, _i32,
                                             ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "pba_paged_decode_ragged": (ctypes.c_int, [_P, _vp, _i32, _vp, _vp, _i32, _vp, _i32,
                                               ctypes.c_float, _vp, _vp, _i32, _vp, _sz, _vp]),
    "pba_expand_block_tables": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp]),
    "pba_pack_block_tables": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "pba_paged_decode_shared_workspace_bytes": (_sz, [_P, _i32, _i32, _i32, _SP]),
    "pba_paged_decode_shared": (ctypes.c_int, [_P, _vp, _i32, _vp, _i32, _vp, _i32, ctypes.c_float,
                                               _vp, _vp, _SP, _vp, _sz, _vp]),
    "pba_paged_decode_shared_append": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                                      _vp, _i32, ctypes.c_float, _vp, _vp, _SP,
                                                      _vp, _sz, _vp]),
    "pba_group_layer_pool": (ctypes.c_int, [_GP, _i32, _P]),
    "pba_kv_append_bundle": (ctypes.c_int, [_GP, _i32, _vp, _vp, _vp, _i64, _vp]),
    "pba_block_copy_bundle": (ctypes.c_int, [_GP, _i32, _vp, _vp, _vp, _vp]),
    "pba_vkv_create": (ctypes.c_int, [ctypes.POINTER(VkvConfig), ctypes.POINTER(_vp)]),
    "pba_vkv_destroy": (ctypes.c_int, [_vp]),
    "pba_vkv_map": (ctypes.c_int, [_vp, _i32, _i64]),
    "pba_vkv_free": (ctypes.c_int, [_vp, _i32, _i32]),
    "pba_vkv_group": (ctypes.c_int, [_vp, _GP, ctypes.POINTER(_i32)]),
    "pba_vkv_capacity": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i64)]),
    "pba_vkv_get_ledgers": (ctypes.c_int, [_vp, ctypes.POINTER(VkvLedgers)]),
    "pba_paged_decode_contiguous": (ctypes.c_int, [_P, _vp, _i32, _vp, _i32, _vp, _i32,
                                                   ctypes.c_float, _vp, _vp, _i32, _vp, _sz, _vp]),
    "pba_paged_decode_noalloc": (ctypes.c_int, [_P, _vp, _i32, _vp, _i32, _vp, _i32, ctypes.c_float,
                                                _vp, _vp, _i32, _vp]),
    "pba_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pba_set_validate": (ctypes.c_int, [ctypes.c_int]),
    "pba_version": (ctypes.c_int, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class PBAError(RuntimeError):
    def __init__(self, call: str, status: int):
        msg = _lib.pba_status_string(status).decode()
        super().__init__(f"{call}: {STATUS.get(status, status)} ({msg})")
        self.status = status


def _check(call: str, status: int) -> None:
    if status != 0:
        raise PBAError(call, status)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass(frozen=True)
class KVPool:
    """One layer's K/V pool: K [NB, H_kv, P, d] (token-major tiles) and
    V [NB, H_kv, d, P] (dim-major tiles), both of the pool dtype."""

    k: torch.Tensor
    v: torch.Tensor
    split_log2: int = 0   # > 0: kernel view, 2^split_log2 kernel blocks per tile

    def __post_init__(self):
        k, v = self.k, self.v
        nb, h, p, d = k.shape
        if v.shape != (nb, h, d, p) or v.dtype != k.dtype or v.device != k.device:
            raise ValueError("V pool must be [num_blocks, H_kv, head_dim, block_size] of K's dtype")
        if k.dtype not in _DTYPES:
            raise TypeError(f"pool dtype {k.dtype} not supported")
        if k.stride(2) != d or k.stride(3) != 1 or v.stride(2) != p or v.stride(3) != 1:
            raise ValueError("pool tiles must be dense ([P][d] for K, [d][P] for V)")
        s = self.split_log2
        if s < 0 or p % (1 << s):
            raise ValueError("split_log2 must split the tile into whole kernel blocks")
        desc = PoolDesc(k.data_ptr(), v.data_ptr(), _DTYPES[k.dtype], nb << s, p >> s, h, d, s,
                        k.stride(0), k.stride(1), v.stride(0), v.stride(1))
        object.__setattr__(self, "_desc", desc)
        object.__setattr__(self, "_ref", ctypes.byref(desc))

    @classmethod
    def empty(cls, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
              dtype=torch.bfloat16, device="cuda") -> "KVPool":
        k = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype, device=device)
        v = torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=dtype, device=device)
        return cls(k, v)

    def kernel_view(self, kernel_block_size: int) -> "KVPool":
        """The same memory exposed as blocks of kernel_block_size tokens
        (allocator block a = kernel blocks a q .. a q + q - 1): for the decode
        calls, with tables from expand_block_tables."""
        q = self.k.shape[2] // kernel_block_size
        if q < 1 or q * kernel_block_size != self.k.shape[2] or q & (q - 1):
            raise ValueError("the kernel block must divide the tile by a power of two")
        return KVPool(self.k, self.v, q.bit_length() - 1)

    @property
    def num_blocks(self) -> int:
        return self.k.shape[0] << self.split_log2

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def block_size(self) -> int:
        return self.k.shape[2] >> self.split_log2

    @property
    def head_dim(self) -> int:
        return self.k.shape[3]

    @property
    def dtype(self):
        return self.k.dtype

    @property
    def device(self):
        return self.k.device

    def desc(self) -> PoolDesc:
        return self._desc


def _require(t: torch.Tensor, name: str, dtype, device, ndim: int):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous rank-{ndim} tensor")


def kv_append(pool: KVPool, slot_mapping: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, stream=None) -> None:
    """Write row i of k_new/v_new [n, H_kv, d] at slot_mapping[i] (int64; < 0 skips)."""
    dev = pool.device
    _require(slot_mapping, "slot_mapping", torch.int64, dev, 1)
    _require(k_new, "k_new", pool.dtype, dev, 3)
    _require(v_new, "v_new", pool.dtype, dev, 3)
    n = slot_mapping.shape[0]
    if k_new.shape != (n, pool.num_kv_heads, pool.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [n_tokens, H_kv, head_dim]")
    _check("pba_kv_append", _lib.pba_kv_append(pool._ref, slot_mapping.data_ptr(), n,
                                               k_new.data_ptr(), v_new.data_ptr(), _stream(stream)))


def block_copy(pool: KVPool, src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Copy whole physical blocks src[k] -> dst[k] (int32 ids), K and V."""
    dev = pool.device
    _require(src, "src", torch.int32, dev, 1)
    _require(dst, "dst", torch.int32, dev, 1)
    if src.shape != dst.shape:
        raise ValueError("src and dst must have the same length")
    _check("pba_block_copy", _lib.pba_block_copy(pool._ref, src.data_ptr(), dst.data_ptr(),
                                                 src.shape[0], _stream(stream)))


def paged_decode_plan(pool: KVPool, num_q_heads: int, batch: int, max_blocks_per_seq: int,
                      partition_tokens: int = 0) -> Tuple[int, int]:
    pt, npart = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("pba_paged_decode_plan", _lib.pba_paged_decode_plan(
        pool._ref, num_q_heads, batch, max_blocks_per_seq, partition_tokens,
        ctypes.byref(pt), ctypes.byref(npart)))
    return pt.value, npart.value


def paged_decode_workspace_bytes(pool: KVPool, num_q_heads: int, batch: int,
                                 max_blocks_per_seq: int, partition_tokens: int = 0) -> int:
    return int(_lib.pba_paged_decode_workspace_bytes(pool._ref, num_q_heads, batch,
                                                     max_blocks_per_seq, partition_tokens))


def paged_decode_plan_ex(pool, num_q_heads: int, batch: int, max_blocks_per_seq: int,
                         partition_tokens: int = 0, seq_lens=None) -> dict:
    """The decomposition the decode calls will use for these arguments, and
    why (host only).  pool: a KVPool or a PoolDesc.  With partition_tokens =
    PARTITIONS_AUTO and the batch's lengths (any int sequence, host side), the
    library chooses; pass the returned "partition_request" to the decode."""
    desc = pool._ref if hasattr(pool, "_ref") else ctypes.byref(pool)
    hint = None
    if seq_lens is not None:
        import numpy as np
        lens = np.asarray(seq_lens, dtype=np.int64)
        hint = ctypes.byref(LengthHint(int(lens.sum()), int(lens.max()) if lens.size else 0, 0))
    info = DecodePlanInfo()
    _check("pba_paged_decode_plan_ex", _lib.pba_paged_decode_plan_ex(
        desc, num_q_heads, batch, max_blocks_per_seq, partition_tokens, hint, ctypes.byref(info)))
    return {"partition_request": info.partition_request,
            "decomposition": DECOMPOSITIONS[info.decomposition],
            "partition_tokens": info.partition_tokens, "num_partitions": info.num_partitions,
            "reason": PLAN_REASONS[info.reason], "fallback": PLAN_REASONS[info.fallback],
            "workspace_bytes": int(info.workspace_bytes)}


def shared_plan_build(tables, seq_lens, block_size: int, group: int, partition_tokens: int = 256,
                      threshold: int = 1, tiles_per_item: int = 4) -> dict:
    """The library's host planner of the shared-prefix decode (host numpy
    arrays in, host arrays out; no device work): the sharing order, the
    plan's items [n, 8] and private ranges [B, 2] (rows in sharing order),
    the chunks [c, 4] and the plan's scalars and ledgers."""
    import numpy as np
    t = np.ascontiguousarray(tables, dtype=np.int32)
    if t.ndim != 2:
        raise ValueError("tables must be [batch, width]")
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, width = t.shape
    if lens.shape != (B,):
        raise ValueError("seq_lens must be [batch]")
    params = SharedPlanParams(block_size, group, partition_tokens, threshold, tiles_per_item, 0)
    info = SharedPlanInfo()
    order = np.zeros(B, dtype=np.int64)
    row_private = np.zeros((B, 2), dtype=np.int32)
    args = (t.ctypes.data if B else None, max(width, 1), lens.ctypes.data if B else None, B,
            ctypes.byref(params))
    _check("pba_shared_plan_build", _lib.pba_shared_plan_build(
        *args, order.ctypes.data if B else None, None, 0,
        row_private.ctypes.data if B else None, None, 0, ctypes.byref(info)))
    items = np.zeros((info.num_items, 8), dtype=np.int32)
    chunks = np.zeros((info.num_chunks, 4), dtype=np.int32)
    _check("pba_shared_plan_build", _lib.pba_shared_plan_build(
        *args, order.ctypes.data if B else None, items.ctypes.data if info.num_items else None,
        info.num_items, row_private.ctypes.data if B else None,
        chunks.ctypes.data if info.num_chunks else None, info.num_chunks, ctypes.byref(info)))
    return {"order": order, "items": items, "row_private": row_private, "chunks": chunks,
            "max_slots": info.max_slots, "private_parts": info.private_parts,
            "private_tokens": info.private_tokens, "partition_tokens": info.partition_tokens,
            "chunk_rows": int(info.chunk_rows), "kv_rows_read": int(info.kv_rows_read),
            "chunk_visits": int(info.chunk_visits), "partial_states": int(info.partial_states)}


_WORKSPACES: "OrderedDict[tuple, torch.Tensor]" = OrderedDict()
_WORKSPACE_CACHE_SIZE = 16


def _torch_stream(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device)
    return stream


def _cached_workspace(device, stream, layout: tuple, need: int) -> torch.Tensor:
    """A zero-filled workspace of ``need`` bytes for one workspace layout,
    cached per (device, stream, layout), least recently used first out.

    The layout (entry point, batch, kv heads, q heads, head_dim, partial-state
    slots) is part of the key: the completion counters occupy the first
    4 * batch * kv_heads bytes, so two layouts of equal size would otherwise
    put one call's counters on the other's partial states.  The buffer is
    allocated and zeroed on the stream the decode runs on, so the zero fill is
    ordered before the first launch that reads it."""
    s = _torch_stream(stream, device)
    key = (str(device), int(s.cuda_stream), layout, need)
    ws = _WORKSPACES.get(key)
    if ws is None:
        with torch.cuda.stream(s):
            ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
        while len(_WORKSPACES) > _WORKSPACE_CACHE_SIZE:
            _WORKSPACES.popitem(last=False)
    else:
        _WORKSPACES.move_to_end(key)
    return ws


def decode_workspace(pool: KVPool, num_q_heads: int, batch: int, max_blocks_per_seq: int,
                     partition_tokens: int = 0, stream=None) -> Optional[torch.Tensor]:
    """A zero-initialised workspace for paged_decode (and its ragged and
    contiguous forms), cached per (device, stream, layout).  The library
    leaves its counters at zero after every call, so one workspace serves
    every call ordered on that stream."""
    need = paged_decode_workspace_bytes(pool, num_q_heads, batch, max_blocks_per_seq,
                                        partition_tokens)
    if need == 0:
        return None
    pt, n_parts = paged_decode_plan(pool, num_q_heads, batch, max_blocks_per_seq,
                                    partition_tokens)
    layout = ("decode", batch, pool.num_kv_heads, num_q_heads, pool.head_dim, pt, n_parts)
    return _cached_workspace(pool.device, stream, layout, need)


def paged_decode(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor,
                 seq_lens: torch.Tensor, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 want_lse: bool = True, partition_tokens: int = 0,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """q [B, H_q, d] (pool dtype), block_tables int32 [B, max_blocks], seq_lens int32 [B].

    Returns (out float32 [B, H_q, d], lse float32 [B, H_q] or None).  A caller
    supplied workspace must be zero-filled before its first use (the library
    keeps it zeroed afterwards); without one, a cached zeroed workspace is used.
    """
    dev = pool.device
    _require(q, "q", pool.dtype, dev, 3)
    _require(block_tables, "block_tables", torch.int32, dev, 2)
    _require(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, Hq, D = q.shape
    if D != pool.head_dim or block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, block_tables, seq_lens and the pool")
    max_blocks = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", torch.float32, dev, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _require(lse, "lse", torch.float32, dev, 2)
    if workspace is None and B > 0:
        workspace = decode_workspace(pool, Hq, B, max_blocks, partition_tokens, stream)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pba_paged_decode", _lib.pba_paged_decode(
        pool._ref, q.data_ptr(), Hq, block_tables.data_ptr(), max_blocks, seq_lens.data_ptr(), B,
        ctypes.c_float(scale), out.data_ptr(), None if lse is None else lse.data_ptr(),
        partition_tokens, ws_ptr, ws_bytes, _stream(stream)))
    return out, lse


def paged_decode_append(pool: KVPool, new_slots: torch.Tensor, k_new: torch.Tensor,
                        v_new: torch.Tensor, q: torch.Tensor, block_tables: torch.Tensor,
                        seq_lens: torch.Tensor, scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        want_lse: bool = True, partition_tokens: int = 0,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    """One decode step: row r's new token (new_slots[r], its last position, or
    negative for none; k_new / v_new [B, H_kv, d]) is appended and the batch
    decoded in one call -- the same result as kv_append then paged_decode."""
    dev = pool.device
    _require(q, "q", pool.dtype, dev, 3)
    _require(block_tables, "block_tables", torch.int32, dev, 2)
    _require(seq_lens, "seq_lens", torch.int32, dev, 1)
    _require(new_slots, "new_slots", torch.int64, dev, 1)
    _require(k_new, "k_new", pool.dtype, dev, 3)
    _require(v_new, "v_new", pool.dtype, dev, 3)
    B, Hq, D = q.shape
    if D != pool.head_dim or block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, block_tables, seq_lens and the pool")
    if new_slots.shape[0] != B or tuple(k_new.shape) != (B, pool.num_kv_heads, D) \
            or k_new.shape != v_new.shape:
        raise ValueError("new_slots [B] and k_new / v_new [B, H_kv, d] must match the batch")
    max_blocks = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", torch.float32, dev, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _require(lse, "lse", torch.float32, dev, 2)
    if workspace is None and B > 0:
        workspace = decode_workspace(pool, Hq, B, max_blocks, partition_tokens, stream)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pba_paged_decode_append", _lib.pba_paged_decode_append(
        pool._ref, new_slots.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), Hq,
        block_tables.data_ptr(), max_blocks, seq_lens.data_ptr(), B, ctypes.c_float(scale),
        out.data_ptr(), None if lse is None else lse.data_ptr(), partition_tokens, ws_ptr,
        ws_bytes, _stream(stream)))
    return out, lse


def paged_decode_noalloc(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor,
                         seq_lens: torch.Tensor, scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         want_lse: bool = True, partition_tokens: int = 0, stream=None):
    """paged_decode through the allocation-free entry point: the library's
    fixed device scratch holds the partial states, so the call allocates no
    device memory when ``out`` (and ``lse``, if wanted) are given.  Calls on
    one GPU share that scratch: calls that overlap in time race."""
    dev = pool.device
    _require(q, "q", pool.dtype, dev, 3)
    _require(block_tables, "block_tables", torch.int32, dev, 2)
    _require(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, Hq, D = q.shape
    if D != pool.head_dim or block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, block_tables, seq_lens and the pool")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", torch.float32, dev, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _require(lse, "lse", torch.float32, dev, 2)
    _check("pba_paged_decode_noalloc", _lib.pba_paged_decode_noalloc(
        pool._ref, q.data_ptr(), Hq, block_tables.data_ptr(), block_tables.shape[1],
        seq_lens.data_ptr(), B, ctypes.c_float(scale), out.data_ptr(),
        None if lse is None else lse.data_ptr(), partition_tokens, _stream(stream)))
    return out, lse


@dataclass(frozen=True)
class SharedPlan:
    """A shared-prefix plan on the device (see ``blocks.shared_plan`` for how a
    caller builds one from its block tables): chunk-first items int32
    [n, 8] and each row's private range int32 [B, 2].  ``private_tokens``
    bounds every row's private positions (0: no bound given); at most 128,
    the library walks four rows' private ranges per work-group."""

    items: torch.Tensor
    row_private: torch.Tensor
    max_slots: int
    partition_tokens: int
    private_parts: int = 0
    private_tokens: int = 0

    def __post_init__(self):
        dev = self.row_private.device
        _require(self.row_private, "row_private", torch.int32, dev, 2)
        _require(self.items, "items", torch.int32, dev, 2)
        if self.items.shape[1] != 8 or self.row_private.shape[1] != 2:
            raise ValueError("items must be [n, 8] and row_private [B, 2]")
        desc = SharedPlanDesc(self.items.shape[0], self.max_slots, self.partition_tokens,
                              self.private_parts,
                              self.items.data_ptr() if self.items.numel() else None,
                              self.row_private.data_ptr(), self.private_tokens, 0)
        object.__setattr__(self, "_desc", desc)
        object.__setattr__(self, "_ref", ctypes.byref(desc))

    @classmethod
    def from_host(cls, host, device) -> "SharedPlan":
        """From a ``blocks.HostSharedPlan`` (numpy arrays)."""
        items = torch.from_numpy(host.items).to(device)
        if items.numel() == 0:
            items = torch.zeros((0, 8), dtype=torch.int32, device=device)
        return cls(items, torch.from_numpy(host.row_private).to(device), host.max_slots,
                   host.partition_tokens, host.private_parts, host.private_tokens)


def paged_decode_shared_workspace_bytes(pool: KVPool, num_q_heads: int, batch: int,
                                        max_blocks_per_seq: int, plan: SharedPlan) -> int:
    return int(_lib.pba_paged_decode_shared_workspace_bytes(pool._ref, num_q_heads, batch,
                                                            max_blocks_per_seq, plan._ref))


def paged_decode_shared(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor,
                        seq_lens: torch.Tensor, plan: SharedPlan, scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        want_lse: bool = True, workspace: Optional[torch.Tensor] = None,
                        stream=None):
    """paged_decode with shared-prefix execution reuse: same arguments and
    results, the plan in place of ``partition_tokens``.  A caller supplied
    workspace must be zero-filled before its first use."""
    dev = pool.device
    _require(q, "q", pool.dtype, dev, 3)
    _require(block_tables, "block_tables", torch.int32, dev, 2)
    _require(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, Hq, D = q.shape
    if D != pool.head_dim or block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, block_tables, seq_lens and the pool")
    if plan.row_private.shape[0] != B:
        raise ValueError("the plan describes another batch")
    max_blocks = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", torch.float32, dev, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _require(lse, "lse", torch.float32, dev, 2)
    if workspace is None and B > 0:
        need = paged_decode_shared_workspace_bytes(pool, Hq, B, max_blocks, plan)
        if need:
            layout = ("shared", B, pool.num_kv_heads, Hq, D, plan.max_slots)
            workspace = _cached_workspace(dev, stream, layout, need)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pba_paged_decode_shared", _lib.pba_paged_decode_shared(
        pool._ref, q.data_ptr(), Hq, block_tables.data_ptr(), max_blocks, seq_lens.data_ptr(), B,
        ctypes.c_float(scale), out.data_ptr(), None if lse is None else lse.data_ptr(),
        plan._ref, ws_ptr, ws_bytes, _stream(stream)))
    return out, lse


def paged_decode_shared_append(pool: KVPool, new_slots: torch.Tensor, k_new: torch.Tensor,
                               v_new: torch.Tensor, q: torch.Tensor, block_tables: torch.Tensor,
                               seq_lens: torch.Tensor, plan: SharedPlan,
                               scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                               workspace: Optional[torch.Tensor] = None, stream=None):
    """One shared-prefix decode step: row r's new token (new_slots[r], its
    last position, inside its private range, or negative for none; k_new /
    v_new [B, H_kv, d], rows in the batch's order) is appended and the batch
    decoded in one call -- the same result as kv_append then
    paged_decode_shared."""
    dev = pool.device
    _require(q, "q", pool.dtype, dev, 3)
    _require(block_tables, "block_tables", torch.int32, dev, 2)
    _require(seq_lens, "seq_lens", torch.int32, dev, 1)
    _require(new_slots, "new_slots", torch.int64, dev, 1)
    _require(k_new, "k_new", pool.dtype, dev, 3)
    _require(v_new, "v_new", pool.dtype, dev, 3)
    B, Hq, D = q.shape
    if D != pool.head_dim or block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, block_tables, seq_lens and the pool")
    if new_slots.shape[0] != B or tuple(k_new.shape) != (B, pool.num_kv_heads, D) \
            or k_new.shape != v_new.shape:
        raise ValueError("new_slots [B] and k_new / v_new [B, H_kv, d] must match the batch")
    if plan.row_private.shape[0] != B:
        raise ValueError("the plan describes another batch")
    max_blocks = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", torch.float32, dev, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _require(lse, "lse", torch.float32, dev, 2)
    if workspace is None and B > 0:
        need = paged_decode_shared_workspace_bytes(pool, Hq, B, max_blocks, plan)
        if need:
            layout = ("shared", B, pool.num_kv_heads, Hq, D, plan.max_slots)
            workspace = _cached_workspace(dev, stream, layout, need)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pba_paged_decode_shared_append", _lib.pba_paged_decode_shared_append(
        pool._ref, new_slots.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), Hq,
        block_tables.data_ptr(), max_blocks, seq_lens.data_ptr(), B, ctypes.c_float(scale),
        out.data_ptr(), None if lse is None else lse.data_ptr(), plan._ref, ws_ptr, ws_bytes,
        _stream(stream)))
    return out, lse


def paged_decode_ragged(pool: KVPool, q: torch.Tensor, block_entries: torch.Tensor,
                        row_offsets: torch.Tensor, seq_lens: torch.Tensor, max_blocks_per_seq: int,
                        scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                        partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                        stream=None):
    """paged_decode over a compact table: row r is block_entries[row_offsets[r] :
    row_offsets[r + 1]] (int32 entries, int64 offsets [B + 1])."""
    dev = pool.device
    _require(q, "q", pool.dtype, dev, 3)
    _require(block_entries, "block_entries", torch.int32, dev, 1)
    _require(row_offsets, "row_offsets", torch.int64, dev, 1)
    _require(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, Hq, D = q.shape
    if D != pool.head_dim or row_offsets.shape[0] != B + 1 or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, row_offsets, seq_lens and the pool")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if workspace is None and B > 0:
        workspace = decode_workspace(pool, Hq, B, max_blocks_per_seq, partition_tokens, stream)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pba_paged_decode_ragged", _lib.pba_paged_decode_ragged(
        pool._ref, q.data_ptr(), Hq, block_entries.data_ptr() if block_entries.numel() else None,
        row_offsets.data_ptr(), max_blocks_per_seq, seq_lens.data_ptr(), B, ctypes.c_float(scale),
        out.data_ptr(), None if lse is None else lse.data_ptr(), partition_tokens, ws_ptr,
        ws_bytes, _stream(stream)))
    return out, lse


def expand_block_tables(tables: torch.Tensor, split_log2: int, stream=None) -> torch.Tensor:
    """Allocator ids -> kernel ids (a -> a q .. a q + q - 1; -1 stays -1); the
    last axis grows q-fold."""
    if tables.dtype != torch.int32 or not tables.is_contiguous():
        raise ValueError("tables must be contiguous int32")
    q = 1 << split_log2
    out = torch.empty(tables.shape[:-1] + (tables.shape[-1] * q,), dtype=torch.int32,
                      device=tables.device)
    _check("pba_expand_block_tables", _lib.pba_expand_block_tables(
        tables.data_ptr() if tables.numel() else None, tables.numel(), split_log2,
        out.data_ptr() if out.numel() else None, _stream(stream)))
    return out


def pack_block_tables(tables: torch.Tensor, row_offsets: torch.Tensor, total: int,
                      stream=None) -> torch.Tensor:
    """Dense [B, width] table -> compact entries (row r at row_offsets[r]);
    ``total`` = row_offsets[B], known to the caller that computed the offsets."""
    _require(tables, "tables", torch.int32, tables.device, 2)
    _require(row_offsets, "row_offsets", torch.int64, tables.device, 1)
    out = torch.empty(max(total, 1), dtype=torch.int32, device=tables.device)
    B, width = tables.shape
    _check("pba_pack_block_tables", _lib.pba_pack_block_tables(
        tables.data_ptr(), B, width, row_offsets.data_ptr(), out.data_ptr(), _stream(stream)))
    return out[:total]


@dataclass(frozen=True)
class KVGroup:
    """One cache group of L layers with one block table per request.

    layer_major: K [L, NB, H_kv, P, d] and V [L, NB, H_kv, d, P]; otherwise
    block major: K [NB, L, H_kv, P, d] and V [NB, L, H_kv, d, P] (one block's
    layers adjacent).  Tiles are dense as in ``KVPool``.
    """

    k: torch.Tensor
    v: torch.Tensor
    layer_major: bool = True

    def __post_init__(self):
        k, v = self.k, self.v
        if k.dim() != 5 or v.dim() != 5:
            raise ValueError("group K and V must be rank 5")
        la, ba = (0, 1) if self.layer_major else (1, 0)
        L, nb, h, p, d = k.shape[la], k.shape[ba], k.shape[2], k.shape[3], k.shape[4]
        want_v = (L, nb, h, d, p) if self.layer_major else (nb, L, h, d, p)
        if tuple(v.shape) != want_v or v.dtype != k.dtype or v.device != k.device:
            raise ValueError(f"V must be {want_v} of K's dtype and device")
        if k.dtype not in _DTYPES:
            raise TypeError(f"pool dtype {k.dtype} not supported")
        if k.stride(3) != d or k.stride(4) != 1 or v.stride(3) != p or v.stride(4) != 1:
            raise ValueError("group tiles must be dense ([P][d] for K, [d][P] for V)")
        pool = PoolDesc(k.data_ptr(), v.data_ptr(), _DTYPES[k.dtype], nb, p, h, d, 0,
                        k.stride(ba), k.stride(2), v.stride(ba), v.stride(2))
        desc = GroupDesc(pool, L, 0, k.stride(la), v.stride(la))
        object.__setattr__(self, "_desc", desc)

    @classmethod
    def empty(cls, layers: int, num_blocks: int, block_size: int, num_kv_heads: int,
              head_dim: int, dtype=torch.bfloat16, device="cuda", layer_major: bool = True):
        lead = (layers, num_blocks) if layer_major else (num_blocks, layers)
        k = torch.empty(lead + (num_kv_heads, block_size, head_dim), dtype=dtype, device=device)
        v = torch.empty(lead + (num_kv_heads, head_dim, block_size), dtype=dtype, device=device)
        return cls(k, v, layer_major)

    @property
    def num_layers(self) -> int:
        return self._desc.num_layers

    @property
    def num_blocks(self) -> int:
        return self._desc.pool.num_blocks

    @property
    def block_size(self) -> int:
        return self._desc.pool.block_size

    @property
    def num_kv_heads(self) -> int:
        return self._desc.pool.num_kv_heads

    @property
    def head_dim(self) -> int:
        return self._desc.pool.head_dim

    @property
    def dtype(self):
        return self.k.dtype

    @property
    def device(self):
        return self.k.device

    def desc(self) -> GroupDesc:
        return self._desc

    def layer(self, layer: int) -> KVPool:
        """Layer ``layer`` as a single-layer pool (views; no copy), for
        paged_decode and the other single-layer calls."""
        if not 0 <= layer < self.num_layers:
            raise IndexError(layer)
        if self.layer_major:
            return KVPool(self.k[layer], self.v[layer])
        return KVPool(self.k[:, layer], self.v[:, layer])

    def layer_desc(self, layer: int) -> PoolDesc:
        """The library's own layer descriptor (pba_group_layer_pool)."""
        out = PoolDesc()
        _check("pba_group_layer_pool", _lib.pba_group_layer_pool(ctypes.byref(self._desc), layer,
                                                                 ctypes.byref(out)))
        return out


def _group_array(groups):
    if not 1 <= len(groups) <= MAX_GROUPS:
        raise ValueError(f"1 to {MAX_GROUPS} groups")
    return (GroupDesc * len(groups))(*[g.desc() for g in groups])


def kv_append_bundle(groups, slot_mappings, k_new, v_new, stream=None) -> None:
    """Write token i into every layer of every group: group g's rows
    k_new[g][i] / v_new[g][i] ([L_g, H_kv, d] each) at slot_mappings[g][i]
    (int64; a token negative in every group is skipped)."""
    G = len(groups)
    if not (len(slot_mappings) == len(k_new) == len(v_new) == G):
        raise ValueError("one slot mapping and one k_new/v_new per group")
    n = slot_mappings[0].shape[0] if G else 0
    for g, grp in enumerate(groups):
        dev = grp.device
        _require(slot_mappings[g], f"slot_mappings[{g}]", torch.int64, dev, 1)
        _require(k_new[g], f"k_new[{g}]", grp.dtype, dev, 4)
        _require(v_new[g], f"v_new[{g}]", grp.dtype, dev, 4)
        shape = (n, grp.num_layers, grp.num_kv_heads, grp.head_dim)
        if slot_mappings[g].shape[0] != n or tuple(k_new[g].shape) != shape or \
                tuple(v_new[g].shape) != shape:
            raise ValueError(f"group {g}: slots [n] and rows {shape} expected")
    arr = _group_array(groups)
    vp = ctypes.c_void_p * G
    _check("pba_kv_append_bundle", _lib.pba_kv_append_bundle(
        arr, G, vp(*[t.data_ptr() for t in slot_mappings]), vp(*[t.data_ptr() for t in k_new]),
        vp(*[t.data_ptr() for t in v_new]), n, _stream(stream)))


def block_copy_bundle(groups, src_blocks, dst_blocks, stream=None) -> None:
    """Copy whole blocks src_blocks[g][k] -> dst_blocks[g][k] (int32) of every
    layer of every group in one launch; the groups' pair counts may differ."""
    G = len(groups)
    if not (len(src_blocks) == len(dst_blocks) == G):
        raise ValueError("one src/dst list per group")
    for g, grp in enumerate(groups):
        dev = grp.device
        _require(src_blocks[g], f"src_blocks[{g}]", torch.int32, dev, 1)
        _require(dst_blocks[g], f"dst_blocks[{g}]", torch.int32, dev, 1)
        if src_blocks[g].shape != dst_blocks[g].shape:
            raise ValueError(f"group {g}: src and dst lengths differ")
    arr = _group_array(groups)
    vp = ctypes.c_void_p * G
    counts = (ctypes.c_int64 * G)(*[t.shape[0] for t in src_blocks])
    _check("pba_block_copy_bundle", _lib.pba_block_copy_bundle(
        arr, G, vp(*[t.data_ptr() for t in src_blocks]), vp(*[t.data_ptr() for t in dst_blocks]),
        counts, _stream(stream)))


class RawPool:
    """A single-layer pool over memory the library manages (a layer of a
    VKVArena): the same calls as ``KVPool`` accept it."""

    def __init__(self, desc: PoolDesc, dtype, device, owner=None):
        self._desc = desc
        self._ref = ctypes.byref(desc)
        self.dtype = dtype
        self.device = device
        self._owner = owner       # keeps the arena alive

    num_blocks = property(lambda self: self._desc.num_blocks)
    block_size = property(lambda self: self._desc.block_size)
    num_kv_heads = property(lambda self: self._desc.num_kv_heads)
    head_dim = property(lambda self: self._desc.head_dim)

    def desc(self) -> PoolDesc:
        return self._desc


class VKVArena:
    """Contiguous virtual K/V for ``num_slots`` request slots of every layer
    (pba_vkv_*): a virtual reservation whose pages are mapped on demand.

    ``map(slot, tokens)`` backs a slot's first rows; ``free(slot, retain)``
    ends its request; the arena acts as a cache group for kv_append_bundle /
    block_copy_bundle, and ``layer(l)`` is the pool of one layer for
    paged_decode_contiguous (slot index, no block table).  Token t of slot r
    has slot id ``slot_ids(r, t)``.
    """

    def __init__(self, layers: int, slots: int, max_tokens: int, num_kv_heads: int,
                 head_dim: int, block_size: int = 16, page_bytes: int = 2 << 20,
                 num_handles: int = 0, dtype=torch.bfloat16, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self.dtype = dtype
        cfg = VkvConfig(_DTYPES[dtype], layers, slots, num_kv_heads, head_dim, block_size,
                        max_tokens, page_bytes, num_handles)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check("pba_vkv_create", _lib.pba_vkv_create(ctypes.byref(cfg), ctypes.byref(h)))
        self._h = h
        self._desc = GroupDesc()
        bps = ctypes.c_int32()
        _check("pba_vkv_group", _lib.pba_vkv_group(h, ctypes.byref(self._desc), ctypes.byref(bps)))
        self.blocks_per_slot = bps.value
        self.num_slots = slots
        self.max_tokens = max_tokens

    num_layers = property(lambda self: self._desc.num_layers)
    num_blocks = property(lambda self: self._desc.pool.num_blocks)
    block_size = property(lambda self: self._desc.pool.block_size)
    num_kv_heads = property(lambda self: self._desc.pool.num_kv_heads)
    head_dim = property(lambda self: self._desc.pool.head_dim)

    def desc(self) -> GroupDesc:
        return self._desc

    def layer(self, layer: int) -> RawPool:
        out = PoolDesc()
        _check("pba_group_layer_pool", _lib.pba_group_layer_pool(ctypes.byref(self._desc), layer,
                                                                 ctypes.byref(out)))
        return RawPool(out, self.dtype, self.device, self)

    def map(self, slot: int, tokens: int) -> None:
        _check("pba_vkv_map", _lib.pba_vkv_map(self._h, slot, tokens))

    def free(self, slot: int, retain: bool = True) -> None:
        _check("pba_vkv_free", _lib.pba_vkv_free(self._h, slot, 1 if retain else 0))

    def capacity(self, slot: int) -> int:
        t = ctypes.c_int64()
        _check("pba_vkv_capacity", _lib.pba_vkv_capacity(self._h, slot, ctypes.byref(t)))
        return t.value

    def ledgers(self) -> dict:
        led = VkvLedgers()
        _check("pba_vkv_get_ledgers", _lib.pba_vkv_get_ledgers(self._h, ctypes.byref(led)))
        return {f: getattr(led, f) for f, _ in led._fields_}

    def slot_ids(self, slot, tokens):
        """Slot ids of (slot, token) pairs for the append calls (numpy or int)."""
        return slot * self.blocks_per_slot * self.block_size + tokens

    def close(self) -> None:
        if getattr(self, "_h", None):
            _check("pba_vkv_destroy", _lib.pba_vkv_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def paged_decode_contiguous(pool, q: torch.Tensor, slot_index: torch.Tensor,
                            blocks_per_slot: int, seq_lens: torch.Tensor,
                            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                            partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                            stream=None):
    """Decode with a request-slot index (int32 [B]) in place of a block table:
    row r reads rows [0, seq_lens[r]) of slot slot_index[r]."""
    dev = pool.device
    _require(q, "q", pool.dtype, dev, 3)
    _require(slot_index, "slot_index", torch.int32, dev, 1)
    _require(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, Hq, D = q.shape
    if D != pool.head_dim or slot_index.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, slot_index, seq_lens and the pool")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", torch.float32, dev, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _require(lse, "lse", torch.float32, dev, 2)
    if workspace is None and B > 0:
        workspace = decode_workspace(pool, Hq, B, blocks_per_slot, partition_tokens, stream)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pba_paged_decode_contiguous", _lib.pba_paged_decode_contiguous(
        pool._ref, q.data_ptr(), Hq, slot_index.data_ptr(), blocks_per_slot, seq_lens.data_ptr(),
        B, ctypes.c_float(scale), out.data_ptr(), None if lse is None else lse.data_ptr(),
        partition_tokens, ws_ptr, ws_bytes, _stream(stream)))
    return out, lse


def set_validate(on: bool) -> bool:
    return bool(_lib.pba_set_validate(1 if on else 0))


def version() -> int:
    return int(_lib.pba_version())
