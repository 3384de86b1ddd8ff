"""Pins for oracle.attention and oracle.pool.gather.

Independent checks: closed forms, brute force with math.fsum/math.exp, torch's
scaled_dot_product_attention in float64 on the CPU (a separate library), and
the invariances the pages fix (physical placement, paging, shared prefixes,
partition merge).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle.allocator import BlockAllocator
from oracle.bits import bf16_bits_to_f64, f32_bits_to_f64
from oracle.pool import BitPool, replay


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def brute_force(q, K, V, scale):
    """Pure-Python loops: one query row, exact-sum denominators."""
    s = [scale * math.fsum(qa * ka for qa, ka in zip(q, k)) for k in K]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    l = math.fsum(p)
    out = [math.fsum(pi * v[c] for pi, v in zip(p, V)) / l for c in range(len(V[0]))]
    return out, m + math.log(l)


def test_bits_conversions():
    # bfloat16 bit patterns with known values.
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3E80, 0x0001], dtype=np.uint16)
    got = bf16_bits_to_f64(bits)
    assert got[:6].tolist() == [1.0, -2.0, 0.0, -0.0, np.inf, 0.25]
    assert got[6] == 2.0 ** -133          # smallest subnormal bfloat16
    nan = bf16_bits_to_f64(np.array([0x7FC1], dtype=np.uint16))
    assert np.isnan(nan[0])
    f = f32_bits_to_f64(np.array([0x3F800000, 0x40490FDB], dtype=np.uint32))
    assert f[0] == 1.0 and f[1] == float(np.float32(np.pi))
    # Agreement with torch's own bfloat16 reinterpretation.
    t = torch.tensor([1.5, -3.25, 1e-3, 65504.0]).to(torch.bfloat16)
    b = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_to_f64(b), t.to(torch.float64).numpy())


def test_closed_forms():
    rng = np.random.default_rng(1)
    T, d = 23, 16
    K, V = _rand(rng, T, d), _rand(rng, T, d)
    q = _rand(rng, 3, d)
    # q = 0 -> every score equal -> mean of the visible V rows.
    O, lse = att.attention_rows(np.zeros((1, d)), K, V, 0.25)
    assert np.allclose(O[0], V.mean(axis=0), atol=1e-15, rtol=0)
    assert abs(lse[0] - math.log(T)) < 1e-14
    # All K rows equal -> mean of V.
    Keq = np.tile(K[:1], (T, 1))
    O, _ = att.attention_rows(q, Keq, V, 0.25)
    assert np.allclose(O, V.mean(axis=0)[None], atol=1e-14, rtol=0)
    # All V rows equal to c -> c.
    c = _rand(rng, d)
    O, _ = att.attention_rows(q, K, np.tile(c, (T, 1)), 0.25)
    assert np.allclose(O, c[None], atol=1e-14, rtol=0)
    # One key -> that value exactly, LSE = its score.
    O, lse = att.attention_rows(q, K[:1], V[:1], 0.25)
    assert np.array_equal(O, np.tile(V[:1], (3, 1)))
    assert np.allclose(lse, 0.25 * (q @ K[0]), atol=1e-15, rtol=0)


def test_brute_force_agreement():
    rng = np.random.default_rng(2)
    for T, d, G in [(1, 4, 1), (2, 3, 2), (7, 8, 4), (35, 64, 1), (40, 5, 3)]:
        K, V, q = _rand(rng, T, d), _rand(rng, T, d), _rand(rng, G, d)
        scale = 1 / math.sqrt(d)
        O, lse = att.attention_rows(q, K, V, scale)
        for g in range(G):
            o, l = brute_force(q[g].tolist(), K.tolist(), V.tolist(), scale)
            assert np.max(np.abs(O[g] - np.array(o))) <= 1e-13
            assert abs(lse[g] - l) <= 1e-13


def test_against_torch_sdpa_float64():
    rng = np.random.default_rng(3)
    for T, d, G in [(16, 64, 1), (9, 128, 4), (64, 128, 8)]:
        K, V, q = _rand(rng, T, d), _rand(rng, T, d), _rand(rng, G, d)
        scale = 1 / math.sqrt(d)
        O, _ = att.attention_rows(q, K, V, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :],
            torch.from_numpy(K)[None, None].expand(1, G, T, d),
            torch.from_numpy(V)[None, None].expand(1, G, T, d), scale=scale)
        assert np.max(np.abs(O - ref[0, :, 0].numpy())) <= 1e-13


def test_partition_merge_equals_monolithic(golden):
    fx = golden("shared_execution.json")["tree"]
    rng = np.random.default_rng(4)
    # The pages' four-sequence tree shape: d_qk = 2, d_v = 3, one head.
    chunks = {n: (_rand(rng, t, fx["d_qk"]), _rand(rng, t, fx["d_v"]))
              for n, (t, _) in fx["chunks"].items()}
    scale = 1 / math.sqrt(fx["d_qk"])
    worst = 0.0
    for path in fx["paths"]:
        q = _rand(rng, 1, fx["d_qk"])
        K = np.concatenate([chunks[c][0] for c in path])
        V = np.concatenate([chunks[c][1] for c in path])
        O, lse = att.attention_rows(q, K, V, scale)
        states = [att.partial_state(q, *chunks[c], scale) for c in path]
        Om, lsem = att.merge_states(states)
        worst = max(worst, np.max(np.abs(O - Om)), abs(lse[0] - lsem[0]))
    # The pages report 2.3e-16 on their fixture; allow a few ulps here.
    assert worst <= 1e-15
    # Long rows, random partition sizes, GQA groups.
    for T, part in [(2049, 512), (1000, 64), (300, 299), (5, 1)]:
        K, V, q = _rand(rng, T, 32), _rand(rng, T, 32), _rand(rng, 4, 32)
        O, lse = att.attention_rows(q, K, V, 0.2)
        Op, lsep = att.partitioned_attention(q, K, V, 0.2, part)
        assert np.max(np.abs(O - Op)) <= 1e-14 and np.max(np.abs(lse - lsep)) <= 1e-13
    assert att.num_partitions(2049, 512) == 5


def test_empty_partition_is_identity():
    rng = np.random.default_rng(5)
    K, V, q = _rand(rng, 10, 4), _rand(rng, 10, 4), _rand(rng, 2, 4)
    empty = att.partial_state(q, K[:0], V[:0], 0.5)
    assert empty.valid == 0
    a = att.partial_state(q, K[:6], V[:6], 0.5)
    b = att.partial_state(q, K[6:], V[6:], 0.5)
    O1, l1 = att.merge_states([a, b])
    O2, l2 = att.merge_states([empty, a, empty, b, empty])
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)
    with pytest.raises(ValueError):
        att.merge_states([empty])


def test_averaging_normalised_outputs_is_wrong():
    """A plausible mistake the merge must not make (0x0BA): it fails this pin."""
    rng = np.random.default_rng(6)
    K, V, q = _rand(rng, 9, 4), _rand(rng, 9, 4), _rand(rng, 1, 4)
    O, _ = att.attention_rows(q, K, V, 1.0)
    Oa, _ = att.attention_rows(q, K[:3], V[:3], 1.0)
    Ob, _ = att.attention_rows(q, K[3:], V[3:], 1.0)
    assert np.max(np.abs(O - 0.5 * (Oa + Ob))) > 1e-3


def _pool_with_placement(order, P=4, H=2, d=6, T=(9, 5, 12), seed=8):
    """Write the same logical rows under a given free-FIFO order."""
    rng = np.random.default_rng(seed)
    nb = len(order)
    a = BlockAllocator(nb, P, free_order=order)
    rids = [a.new_request() for _ in T]
    for r, t in zip(rids, T):
        a.prefill(r, t)
    n_w = sum(T)
    # Finite bfloat16 with |x| < 2: sign bit plus an exponent field below 0x80.
    k_rows = rng.integers(0, 1 << 16, size=(n_w, H, d), dtype=np.uint16) & 0xBFFF
    v_rows = rng.integers(0, 1 << 16, size=(n_w, H, d), dtype=np.uint16) & 0x3FFF
    pool = BitPool(np.full((nb, H, P, d), 0x7FC1, np.uint16),
                   np.full((nb, H, d, P), 0x7FC1, np.uint16), "bf16")
    replay(pool, a.trace, k_rows, v_rows)
    q = rng.integers(0, 1 << 16, size=(len(T), 2 * H, d), dtype=np.uint16) & 0x3FFF
    return pool, q, [a.table(r) for r in rids], list(T)


def test_placement_invariance_and_paged_equals_contiguous():
    nb = 16
    rng = np.random.default_rng(9)
    outs = []
    for _ in range(3):
        pool, q, tables, lens = _pool_with_placement(rng.permutation(nb).tolist())
        out, lse = att.paged_decode(pool, q, tables, lens, 0.4)
        assert np.all(np.isfinite(out))         # NaN-poisoned padding never read
        outs.append((out, lse))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
    # Contiguous placement: identity free order; same answer bit for bit.
    pool, q, tables, lens = _pool_with_placement(list(range(nb)))
    assert tables[0] == [0, 1, 2]
    out, lse = att.paged_decode(pool, q, tables, lens, 0.4)
    assert np.array_equal(out, outs[0][0])


def test_shared_prefix_equals_private_copies():
    P, H, d = 4, 1, 5
    rng = np.random.default_rng(10)
    prefix, suffix = 10, [3, 0, 6]
    rows = rng.integers(0, 1 << 16, size=(prefix + sum(suffix) + 5, H, d), dtype=np.uint16) & 0x3FFF
    # Shared: one prefix, forked.
    a = BlockAllocator(32, P, free_order=rng.permutation(32))
    p = a.new_request()
    a.prefill(p, prefix)
    kids = [a.fork(p) for _ in suffix]
    for c, s in zip(kids, suffix):
        a.prefill(c, s)
    # Private: every request writes its own copy of the prefix.
    b = BlockAllocator(64, P, free_order=rng.permutation(64))
    priv = [b.new_request() for _ in suffix]
    for r, s in zip(priv, suffix):
        b.prefill(r, prefix + s)
    # Row values: prefix rows are the same for every request.
    def rows_for(trace, private):
        out = []
        cursor = {r: 0 for r in range(100)}
        for op in trace:
            if op[0] != "write":
                continue
            rid, t = op[1], op[2]
            if t < prefix:
                out.append(rows[t])
            else:
                k = (priv.index(rid) if private else kids.index(rid))
                out.append(rows[prefix + sum(suffix[:k]) + (t - prefix)])
        return np.stack(out)
    pool_a = BitPool(np.full((32, H, P, d), 0x7FC1, np.uint16),
                     np.full((32, H, d, P), 0x7FC1, np.uint16), "bf16")
    ra = rows_for(a.trace, False)
    replay(pool_a, a.trace, ra, ra)
    pool_b = BitPool(np.full((64, H, P, d), 0x7FC1, np.uint16),
                     np.full((64, H, d, P), 0x7FC1, np.uint16), "bf16")
    rb = rows_for(b.trace, True)
    replay(pool_b, b.trace, rb, rb)
    q = rng.integers(0, 1 << 16, size=(3, H, d), dtype=np.uint16) & 0x3FFF
    lens = [prefix + s for s in suffix]
    oa, la = att.paged_decode(pool_a, q, [a.table(c) for c in kids], lens, 0.3)
    ob, lb = att.paged_decode(pool_b, q, [b.table(r) for r in priv], lens, 0.3)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_gqa_equals_mha_with_repeated_kv():
    """Convention pin: query head i reads kv head i // G."""
    rng = np.random.default_rng(11)
    P, Hkv, G, d, T = 4, 2, 3, 6, 7
    k = rng.integers(0, 1 << 16, size=(4, Hkv, P, d), dtype=np.uint16) & 0x3FFF
    v = rng.integers(0, 1 << 16, size=(4, Hkv, d, P), dtype=np.uint16) & 0x3FFF
    q = rng.integers(0, 1 << 16, size=(1, Hkv * G, d), dtype=np.uint16) & 0x3FFF
    gqa = att.paged_decode(BitPool(k, v, "bf16"), q, [[2, 0]], [T], 0.5)[0]
    krep, vrep = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    mha = att.paged_decode(BitPool(krep, vrep, "bf16"), q, [[2, 0]], [T], 0.5)[0]
    # Equal up to the order BLAS sums a G-row block versus single rows.
    assert np.max(np.abs(gqa - mha)) <= 1e-15
    # A transposed head map (query head i reading kv head i mod H_kv) differs.
    kalt = np.stack([k[:, i % Hkv] for i in range(Hkv * G)], axis=1)
    valt = np.stack([v[:, i % Hkv] for i in range(Hkv * G)], axis=1)
    alt = att.paged_decode(BitPool(kalt, valt, "bf16"), q, [[2, 0]], [T], 0.5)[0]
    assert np.max(np.abs(gqa - alt)) > 1e-6


def test_tail_rule_reads_only_visible_rows():
    """gather returns T rows; NaN rows beyond T (same block) are never read."""
    P, d = 16, 4
    k = np.full((3, 1, P, d), 0x7FC1, np.uint16)
    v = np.full((3, 1, d, P), 0x7FC1, np.uint16)
    k[2, 0, :3] = 0x3F80
    v[2, 0, :, :3] = 0x4000
    k[0, 0, :] = 0x3F80
    v[0, 0, :, :] = 0x4000
    pool = BitPool(k, v, "bf16")
    for T in (1, 3, 16, 19):
        table = [2] if T <= 3 else [0, 2]
        K, V = pool.gather(table, T, 0)
        assert K.shape == (T, d) and np.all(np.isfinite(K)) and np.all(V == 2.0)
