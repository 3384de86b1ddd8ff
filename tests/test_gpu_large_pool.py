"""GPU: a pool whose K and V tensors each pass 2^31 elements.

Block ids are 32-bit, but a block's element offset (id * stride) is not: the
top blocks of this pool start past 2^31 elements, so every address step --
the append's slot -> (block, offset), the copy's tiles, each decode path's
table lookups -- must widen the id before it multiplies ("Cache Concepts:
Prefix Matching vs. Storage", int64 widening of page ids).  Rows live in the
top blocks (and one at block 0), so a 32-bit product would land far from
them.  The pool is never mirrored on the host: the expected bytes and
outputs come from the rows written and the binary64 oracle.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from harness import to_bits, to_device
from oracle import attention as att
from oracle.bits import bits_to_f64
from test_gpu_parity import pba  # noqa: F401

pytestmark = pytest.mark.gpu

NB, P, H, G, D = 40000, 64, 8, 4, 128  # K and V: 40000 x 8 x 64 x 128 bf16, 5.2 GB each
BAL = -1


def say(*msg):
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def test_pool_beyond_2g_elements(pba, gpu):
    assert NB * H * P * D > 2 ** 31 and (NB - 13) * H * P * D > 2 ** 31
    say("large pool", NB, "blocks,", NB * H * P * D * 2 >> 20, "MiB per tensor")
    pool = pba.KVPool.empty(NB, P, H, D, torch.bfloat16, gpu)
    lens = np.array([700, 130, 65], dtype=np.int32)
    rows = [list(range(NB - 11, NB)), [20000, NB - 12, 33333], [0, NB - 13]]
    mb = max(len(r) for r in rows)
    tables = np.zeros((len(rows), mb), dtype=np.int32)
    for r, ids in enumerate(rows):
        tables[r, :len(ids)] = ids
    # Token t of row r goes to slot table[r][t // P] * P + t % P.
    slots = np.concatenate([[rows[r][t // P] * P + t % P for t in range(int(T))]
                            for r, T in enumerate(lens)]).astype(np.int64)
    first = np.concatenate([[0], np.cumsum(lens)])
    kb = wl.normal_bits(20261202 + 9100, (int(lens.sum()), H, D), "bf16")
    vb = wl.normal_bits(20261202 + 9101, (int(lens.sum()), H, D), "bf16")
    pba.kv_append(pool, torch.from_numpy(slots).to(gpu), to_device(kb, "bf16", gpu),
                  to_device(vb, "bf16", gpu))
    torch.cuda.synchronize()

    # The top block holds tokens 640..699 of row 0: K [H][P][D], V [H][D][P].
    got_k = to_bits(pool.k[NB - 1])
    got_v = to_bits(pool.v[NB - 1])
    for t in range(640, 700):
        assert np.array_equal(got_k[:, t - 640, :], kb[first[0] + t]), t
        assert np.array_equal(got_v[:, :, t - 640], vb[first[0] + t]), t
    # Row 2's first token sits at block 0 (the low end of the same tensors).
    assert np.array_equal(to_bits(pool.k[0])[:, 0, :], kb[first[2]])

    # A whole-block copy from the top of the pool to block 1 and back up to a
    # free top block: bit for bit in both directions.
    say("large pool copies")
    pba.block_copy(pool, torch.tensor([NB - 1], dtype=torch.int32, device=gpu),
                   torch.tensor([1], dtype=torch.int32, device=gpu))
    pba.block_copy(pool, torch.tensor([NB - 2], dtype=torch.int32, device=gpu),
                   torch.tensor([NB - 20], dtype=torch.int32, device=gpu))
    torch.cuda.synchronize()
    assert torch.equal(pool.k[1].view(torch.int16), pool.k[NB - 1].view(torch.int16))
    assert torch.equal(pool.v[1].view(torch.int16), pool.v[NB - 1].view(torch.int16))
    assert torch.equal(pool.k[NB - 20].view(torch.int16), pool.k[NB - 2].view(torch.int16))
    assert torch.equal(pool.v[NB - 20].view(torch.int16), pool.v[NB - 2].view(torch.int16))

    qb = wl.normal_bits(20261202 + 9102, (len(rows), H * G, D), "bf16")
    q = to_device(qb, "bf16", gpu)
    scale = 1.0 / math.sqrt(D)
    qf = bits_to_f64(qb, "bf16")
    kf = bits_to_f64(kb, "bf16")
    vf = bits_to_f64(vb, "bf16")
    ref = np.zeros((len(rows), H * G, D))
    ref_lse = np.zeros((len(rows), H * G))
    for r, T in enumerate(lens):
        for h in range(H):
            o, l = att.attention_rows(qf[r, h * G:(h + 1) * G], kf[first[r]:first[r] + T, h],
                                      vf[first[r]:first[r] + T, h], scale)
            ref[r, h * G:(h + 1) * G] = o
            ref_lse[r, h * G:(h + 1) * G] = l
    tab = torch.from_numpy(tables).to(gpu)
    ln = torch.from_numpy(lens).to(gpu)
    for pt in (0, 256, BAL):
        say("large pool decode, partition_tokens", pt)
        out, lse = pba.paged_decode(pool, q, tab, ln, scale, partition_tokens=pt)
        torch.cuda.synchronize()
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= 2e-3, pt
        assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 2e-3, pt
    del pool
    torch.cuda.empty_cache()
