"""Row, block and byte ledgers the pages print.

Test infrastructure only (see ``oracle/__init__.py``).  Each function names the
passage of "M5.3 - KV Memory Layout and Exact Reuse" (P1) or "7. Memory
Management and Local Model State" (P3) whose formula it writes out.
"""
from __future__ import annotations

from typing import Dict, Mapping, Sequence, Tuple


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def row_bytes(layers: int, kv_heads: int, head_dim: int, bytes_k: int, bytes_v: int) -> int:
    """B_row = L * H_kv * d_h * (b_K + b_V)   (P1 0x02A)."""
    return layers * kv_heads * head_dim * (bytes_k + bytes_v)


def blocks_needed(T: int, P: int) -> int:
    """N_r = ceil(T_r / P)   (P1 0x02C, 0x09B; P3 "Logical tokens, physical blocks")."""
    return ceil_div(T, P)


def last_block_rows(T: int, P: int) -> int:
    """Valid rows of the last logical block: T mod P, or P when that is 0 (P1 0x0A)."""
    if T <= 0:
        raise ValueError("empty request has no last block")
    return T % P or P


def request_tail_slots(T: int, P: int) -> int:
    """W_r = N_r P - T_r   (P1 0x09B)."""
    return blocks_needed(T, P) * P - T


def request_view_ledger(lengths: Sequence[int], P: int) -> Dict[str, int]:
    """N_ref = sum N_r; request-view tail = N_ref P - sum T_r   (P1 0x02C)."""
    n_ref = sum(blocks_needed(T, P) for T in lengths)
    return {"refs": n_ref, "slots": n_ref * P, "logical_rows": sum(lengths),
            "tail_slots": n_ref * P - sum(lengths)}


def unique_ledger(tables: Mapping[int, Sequence[int]], lengths: Mapping[int, int],
                  P: int) -> Dict[str, object]:
    """Union of physical ids and the rows materialised in each (P1 0x02D).

    v_p is the largest number of rows of block p that any referencing request
    makes visible (exact-prefix families materialise the longest view).
    """
    rows: Dict[int, int] = {}
    for rid, table in tables.items():
        T = lengths[rid]
        for j, b in enumerate(table):
            visible = P if j < len(table) - 1 else last_block_rows(T, P)
            rows[b] = max(rows.get(b, 0), visible)
    return {"ids": sorted(rows), "unique": len(rows),
            "materialized_rows": sum(rows.values()),
            "tail_slots": sum(P - v for v in rows.values())}


def rect_ledger(lengths: Sequence[int], reserved: Sequence[int]) -> Dict[str, int]:
    """Rectangular reservation: reserved rows and slack (P1 0x02B)."""
    return {"logical_rows": sum(lengths), "reserved_rows": sum(reserved),
            "slack_rows": sum(reserved) - sum(lengths)}


def table_cells(lengths: Sequence[int], P: int) -> Dict[str, int]:
    """Dense staging table: N_table = B n_max, N_used = sum n_r, N_pad   (P1 0x0AB)."""
    n = [blocks_needed(T, P) for T in lengths]
    n_max = max(n) if n else 0
    return {"table": len(n) * n_max, "used": sum(n), "pad": len(n) * n_max - sum(n),
            "n_max": n_max}


def decode_partitions(T: int, P_k: int, P_part: int) -> Dict[str, int]:
    """N_seq-blocks = ceil(T/P_k); N_parts = ceil(T/P_part); N_blocks/part = P_part/P_k.

    P_k must divide P_part (P1 0x0A).
    """
    if P_part % P_k:
        raise ValueError("kernel block size must divide the partition size")
    return {"seq_blocks": ceil_div(T, P_k), "parts": ceil_div(T, P_part),
            "blocks_per_part": P_part // P_k}


def cow_cost(valid_tail_rows: int, bundle_row_bytes: int) -> Dict[str, float]:
    """B_copy = r B_row; traffic = 2 B_copy + B_row; amplification 2r + 1 (P1 0x05A)."""
    copy = valid_tail_rows * bundle_row_bytes
    traffic = 2 * copy + bundle_row_bytes
    return {"copy_payload": copy, "read_plus_write": 2 * copy, "append_write": bundle_row_bytes,
            "traffic": traffic, "amplification": traffic / bundle_row_bytes}


def cow_capacity(shared_tokens: int, P: int, B_row: int) -> Dict[str, object]:
    """r = shared mod P; copy R+W = 2 r B_row; destination P B_row; A = P / r (P1 0x09C).

    r == 0: the prefix ends on a block boundary and no copy is made.
    """
    r = shared_tokens % P
    if r == 0:
        return {"r": 0, "copy": False, "copy_rw_bytes": 0, "dst_bytes": 0,
                "capacity_amplification": None}
    return {"r": r, "copy": True, "copy_rw_bytes": 2 * r * B_row, "dst_bytes": P * B_row,
            "capacity_amplification": P / r}


def expected_tail_slots(P: int) -> float:
    """E[P - J] = (P - 1) / 2 for J uniform on {1..P}   (P1 0x02G)."""
    return (P - 1) / 2


def shared_prefix_rows(B: int, S: int, U: Sequence[int]) -> Dict[str, int]:
    """N_logical = B S + sum U_r; N_unique = S + sum U_r; N_saved = (B - 1) S (P1 0x0BI)."""
    return {"logical": B * S + sum(U), "unique": S + sum(U), "saved": (B - 1) * S}


def chunk_tree_ledger(chunks: Mapping[str, Tuple[int, Tuple[int, int]]],
                      paths: Sequence[Sequence[str]], threshold: int,
                      row_bytes_kv: int, partial_row_bytes: int) -> Dict[str, int]:
    """Logical pairs, unique rows, saved reads, partial rows and bytes (P1 0x0BE).

    chunks: name -> (rows T_c, coverage half-open interval); paths: chunk names
    of each sequence; a chunk is materialised chunk-first when its coverage
    exceeds ``threshold``.
    """
    logical = sum(chunks[c][0] for path in paths for c in path)
    unique = sum(t for t, _ in chunks.values())
    partial = sum(e - b for t, (b, e) in chunks.values() if e - b > threshold)
    return {"logical_pairs": logical, "unique_rows": unique, "saved": logical - unique,
            "baseline_bytes": logical * row_bytes_kv, "shared_bytes": unique * row_bytes_kv,
            "partial_rows": partial, "partial_bytes": partial * partial_row_bytes}


def kernel_block_ids(alloc_ids: Sequence[int], P_a: int, P_k: int):
    """Allocator block a -> kernel blocks {a q, ..., a q + q - 1}, q = P_a / P_k (P1 0x0AC)."""
    if P_a % P_k:
        raise ValueError("kernel block size must divide the allocator block size")
    q = P_a // P_k
    return [a * q + i for a in alloc_ids for i in range(q)]
