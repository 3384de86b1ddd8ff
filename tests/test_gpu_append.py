"""GPU: kv_append's slot patterns, bit for bit against a host scatter of the
same bits (the pool layout of the ABI: K [block][head][P][d], V
[block][head][d][P]; slot s -> block s // P, offset s % P).

Appends of 1024 tokens or more move the V rows in blocks of 16 /
sizeof(scalar) consecutive tokens, stored as one 16-byte run per dim when the
block's slots are consecutive and start at a multiple of that size, scalar
by scalar otherwise; smaller appends move one token's piece per thread.  The
token counts cover both, and the slot patterns mix both block cases: a
prefill of aligned runs, runs starting off the alignment, runs with skipped
(negative) slots, runs broken by a block boundary, scattered decode slots,
token counts that leave a partial last block, bf16 and fp32 pools, block
sizes 16 to 256 and head dims 64 and 128.  NaN payloads must survive.
Every case prints its name before its GPU work."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def say(*msg):
    print("[case]", *msg, flush=True)


def host_scatter(kb, vb, slots, knew, vnew, P):
    """The expected pools: each non-negative slot's K row and V column."""
    kb, vb = kb.copy(), vb.copy()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), P)
        kb[b, :, o, :] = knew[i]
        vb[b, :, :, o] = vnew[i]
    return kb, vb


def slot_pattern(name, n, P, nb, rng):
    if name == "prefill":          # consecutive slots over whole blocks in a seeded order
        blocks = rng.permutation(nb)[: -(-n // P)]
        return (blocks[:, None] * P + np.arange(P)).reshape(-1)[:n]
    if name == "prefill_offset":   # a run that starts 3 positions into its first block
        blocks = rng.permutation(nb)[: -(-(n + 3) // P)]
        return (blocks[:, None] * P + np.arange(P)).reshape(-1)[3:n + 3]
    if name == "prefill_skips":    # aligned runs with some slots skipped
        s = slot_pattern("prefill", n, P, nb, rng).copy()
        s[rng.random(n) < 0.2] = -1
        return s
    if name == "block_breaks":     # runs of 8 that restart in another block every 5 tokens
        blocks = rng.permutation(nb)
        return np.array([blocks[i // 5] * P + (i % 5) for i in range(n)])
    if name == "scattered":        # one token per request, decode style
        return rng.choice(nb * P, size=n, replace=False)
    raise ValueError(name)


CASES = [("bf16", 16, 128, 8), ("bf16", 64, 128, 8), ("bf16", 256, 64, 2), ("bf16", 32, 64, 3),
         ("f32", 16, 64, 2), ("f32", 64, 128, 1)]


@pytest.mark.parametrize("pattern", ["prefill", "prefill_offset", "prefill_skips", "block_breaks",
                                     "scattered"])
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("n", [1, 7, 8, 63, 64, 517, 1024, 2053])
def test_append_slot_patterns(gpu, pattern, case, n):
    import block_table_attention_amd as pba

    dt, P, d, H = CASES[case]
    rng = np.random.default_rng(20261202 + 9000 + case * 100 + n)
    nb = max(8, 2 * (-(-(n + 8) // P)) + 4, n // 5 + 2)
    slots = slot_pattern(pattern, n, P, nb, rng).astype(np.int64)
    say(pattern, dt, "P", P, "d", d, "H", H, "n", n, "blocks", nb)
    bits = np.uint16 if dt == "bf16" else np.uint32
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ibits = torch.int16 if dt == "bf16" else torch.int32
    kb = rng.integers(0, np.iinfo(bits).max, size=(nb, H, P, d), dtype=bits)
    vb = rng.integers(0, np.iinfo(bits).max, size=(nb, H, d, P), dtype=bits)
    knew = rng.integers(0, np.iinfo(bits).max, size=(n, H, d), dtype=bits)
    vnew = rng.integers(0, np.iinfo(bits).max, size=(n, H, d), dtype=bits)
    if n > 1:  # NaN payloads (all exponent bits set) survive the copies
        knew[0, 0, :2] = 0x7FC1 if dt == "bf16" else 0x7FC00001
        vnew[n - 1, H - 1, -2:] = 0xFFC3 if dt == "bf16" else 0xFFC00003

    def dev(a):
        return torch.from_numpy(a.view(np.int16 if dt == "bf16" else np.int32)).to(gpu).view(tdt)

    pool = pba.KVPool(dev(kb), dev(vb))
    pba.kv_append(pool, torch.from_numpy(slots).to(gpu), dev(knew), dev(vnew))
    torch.cuda.synchronize()
    ek, ev = host_scatter(kb, vb, slots, knew, vnew, P)
    assert np.array_equal(pool.k.view(ibits).cpu().numpy().view(bits), ek)
    assert np.array_equal(pool.v.view(ibits).cpu().numpy().view(bits), ev)
