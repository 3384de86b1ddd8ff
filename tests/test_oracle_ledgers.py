"""Pins for oracle.ledgers against the values the pages print."""
import numpy as np

from oracle import ledgers as L
from oracle.allocator import BlockAllocator


def test_nested_family_ledger(golden):
    fx = golden("nested_ledger.json")
    lay, e = fx["layout"], fx["expect"]
    B_row = L.row_bytes(lay["layers"], lay["kv_heads"], lay["head_dim"], lay["bytes_k"], lay["bytes_v"])
    assert B_row == e["row_bytes"] == 65536
    P = lay["P"]
    lengths = fx["requests"]
    lens = list(lengths.values())
    rv = L.request_view_ledger(lens, P)
    assert rv["logical_rows"] == e["logical_rows"] and rv["logical_rows"] * B_row == e["logical_bytes"]
    assert rv["refs"] == e["refs"] == 6
    assert rv["slots"] == e["request_view_slots"] and rv["slots"] * B_row == e["request_view_bytes"]
    assert rv["tail_slots"] == e["request_view_tail_slots"] == 22
    assert rv["tail_slots"] * B_row == e["request_view_tail_bytes"]
    rect = L.rect_ledger(lens, list(fx["reserved_rows"].values()))
    assert rect["reserved_rows"] * B_row == e["reserved_bytes"]
    assert rect["slack_rows"] * B_row == e["slack_bytes"]
    u = L.unique_ledger(fx["tables"], lengths, P)
    assert u["ids"] == e["unique_ids"] and u["unique"] == 3
    assert u["materialized_rows"] == e["unique_materialized_rows"] == 33
    assert u["materialized_rows"] * B_row == e["unique_materialized_bytes"]
    assert u["unique"] * P == e["unique_slots"] and u["unique"] * P * B_row == e["unique_capacity_bytes"]
    assert u["tail_slots"] == e["unique_tail_slots"] == 15
    assert u["tail_slots"] * B_row == e["unique_tail_bytes"]
    assert (rv["logical_rows"] - u["materialized_rows"]) * B_row == e["dedup_payload_bytes"]
    # Checked identities printed in the section.
    assert e["reserved_bytes"] == e["logical_bytes"] + e["slack_bytes"]
    assert e["request_view_bytes"] == e["logical_bytes"] + e["request_view_tail_bytes"]
    assert e["unique_capacity_bytes"] == e["unique_materialized_bytes"] + e["unique_tail_bytes"]
    assert e["pool_blocks"] - u["unique"] == e["idle_blocks"]


def test_nested_family_through_the_allocator(golden):
    """The same family built by fork + truncation-free prefixes: A=33, B=25, C=16."""
    fx = golden("nested_ledger.json")
    a = BlockAllocator(8, 16, free_order=[100 - 100 + i for i in range(8)])
    A = a.new_request()
    a.prefill(A, 33)
    # B and C view exact prefixes of A: map the first ceil(T/P) blocks.
    tables = {"A": a.table(A), "B": a.table(A)[:2], "C": a.table(A)[:1]}
    u = L.unique_ledger(tables, fx["requests"], 16)
    assert u["unique"] == 3 and u["tail_slots"] == 15 and u["materialized_rows"] == 33
    assert a.n_live() == fx["expect"]["live_blocks"] and a.n_free() == fx["expect"]["idle_blocks"]


def test_block_size_sweep(golden):
    fx = golden("block_size_sweep.json")
    lens, B_row = fx["lengths"], fx["row_bytes"]
    for P_s, e in fx["expect"].items():
        P = int(P_s)
        n_unique = L.blocks_needed(max(lens), P)
        tail = n_unique * P - max(lens)
        assert tail == e["unique_tail_slots"] and tail * B_row == e["unique_tail_bytes"]
        if "descriptors" in e:
            assert fx["pool_slots"] // P == e["descriptors"]
            assert L.request_view_ledger(lens, P)["refs"] == e["map_entries"]


def test_p3_examples(golden):
    fx = golden("p3_examples.json")
    t = fx["tokens35"]
    assert L.blocks_needed(t["T"], t["P"]) == t["blocks"]
    assert L.last_block_rows(t["T"], t["P"]) == t["tail_rows"]
    h = fx["tokens100"]
    assert L.blocks_needed(100, 16) == h["P16_blocks"]
    assert L.blocks_needed(100, 256) == h["P256_blocks"]
    assert L.request_tail_slots(100, 256) == h["P256_unused"]
    assert max(L.request_tail_slots(T, 16) for T in range(1, 200)) == h["P16_max_unused"]
    assert L.last_block_rows(32, 16) == 16 and L.last_block_rows(33, 16) == 1


def test_cow_costs(golden):
    fx = golden("cow_trace.json")
    c = fx["cost"]
    got = L.cow_cost(c["valid_tail_rows"], c["bundle_row_bytes"])
    for k, v in c["expect"].items():
        if k in got:
            assert got[k] == v, k
    assert 16 * c["bundle_row_bytes"] == c["expect"]["new_capacity_bytes"]
    s = fx["shared20"]
    cap = L.cow_capacity(s["shared_tokens"], s["P"], 1)
    assert cap["r"] == s["r"] and cap["copy"] and cap["capacity_amplification"] == 16 / 4
    assert cap["copy_rw_bytes"] == 8 and cap["dst_bytes"] == 16
    assert not L.cow_capacity(s["shared_tokens"], s["boundary_P"], 1)["copy"]


def test_decode_partitions(golden):
    fx = golden("decode_partitions.json")
    for P in fx["block_sizes"]:
        got = L.decode_partitions(fx["T"], P, fx["P_part"])
        assert got["parts"] == fx["expect"]["parts"] == 5
        assert got["seq_blocks"] == fx["expect"]["seq_blocks"][str(P)]
        assert got["blocks_per_part"] == fx["expect"]["blocks_per_part"][str(P)]


def test_table_cells_formula():
    # Ragged lengths [64, 63, 17, 1] (the pages' fixture table did not survive
    # extraction; the cells are recomputed from the printed formula).
    got = L.table_cells([64, 63, 17, 1], 16)
    assert got == {"table": 16, "used": 4 + 4 + 2 + 1, "pad": 16 - 11, "n_max": 4}


def test_expected_tail_statistics():
    assert L.expected_tail_slots(16) == 7.5
    rng = np.random.default_rng(12)
    T = rng.integers(1, 100_000, size=200_000)
    mean = np.mean([(-(-t // 16)) * 16 - t for t in T[:20000]])
    assert abs(mean - 7.5) < 0.15


def test_shared_execution_ledgers(golden):
    fx = golden("shared_execution.json")
    t = fx["tree"]
    chunks = {n: (rows, tuple(cov)) for n, (rows, cov) in t["chunks"].items()}
    row = (t["d_qk"] + t["d_v"]) * t["bytes"]
    prow = t["d_v"] * t["bytes"] + 2 * t["state_bytes"]
    got = L.chunk_tree_ledger(chunks, t["paths"], t["threshold"], row, prow)
    e = t["expect"]
    assert row == e["row_bytes"] and prow == e["partial_row_bytes"]
    for k in ("logical_pairs", "unique_rows", "saved", "baseline_bytes", "shared_bytes",
              "partial_rows", "partial_bytes"):
        assert got[k] == e[k], k
    l10 = fx["loop10"]
    got = L.shared_prefix_rows(l10["B"], l10["S"], l10["U"])
    e = l10["expect"]
    assert (got["logical"], got["unique"], got["saved"]) == (e["logical"], e["unique"], e["saved"])
    assert got["logical"] * l10["row_bytes"] == e["baseline_bytes"]
    assert got["unique"] * l10["row_bytes"] == e["shared_bytes"]
    assert got["saved"] * l10["row_bytes"] == e["saved_bytes"]
    ks = fx["kernel_split"]
    assert L.kernel_block_ids(ks["alloc_ids"], ks["P_a"], ks["P_k"]) == ks["expect"]
