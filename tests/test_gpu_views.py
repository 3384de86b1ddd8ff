"""GPU parity of kernel views of allocator pools and compact (ragged) tables.

* pba_expand_block_tables and pba_pack_block_tables are bit exact against the
  oracle's expansion and packing ("M5.3", 0x0AC and 0x0AB).
* Decoding through a kernel view (allocator blocks of P_a rows read as kernel
  blocks of P_k rows, tables expanded by the library) and through a compact
  table gives the oracle's result within 2e-3, and is bitwise equal to the
  dense allocator-view decode: the kernel sees the same tokens in the same
  order and the same partition plan.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from harness import execute, gpu_pool, gpu_replay, oracle_pool, to_device
from oracle import attention as att
from oracle import views

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


@pytest.mark.parametrize("split", [1, 2, 4])
def test_expand_bit_exact(pba, gpu, split):
    rng = np.random.default_rng(900 + split)
    tables = rng.integers(0, 5000, size=(37, 23)).astype(np.int32)
    tables[rng.random(tables.shape) < 0.2] = -1
    say("expand", tables.shape, "split", split)
    got = pba.expand_block_tables(torch.from_numpy(tables).to(gpu), split).cpu().numpy()
    q = 1 << split
    for r in range(tables.shape[0]):
        want = []
        for a in tables[r]:
            want.extend([-1] * q if a < 0 else views.expand_table([int(a)], q, 1))
        assert got[r].tolist() == want


def test_pack_bit_exact(pba, gpu):
    w = wl.lognormal(16, batch=64)
    ex = execute(w)
    say("pack", ex.tables.shape)
    entries, offsets = views.pack_ragged(ex.tables, ex.seq_lens, 16)
    got = pba.pack_block_tables(torch.from_numpy(ex.tables).to(gpu),
                                torch.from_numpy(offsets).to(gpu), int(offsets[-1]))
    assert np.array_equal(got.cpu().numpy(), entries)


def _setup(w, device):
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    pool = gpu_pool(ex, device)
    gpu_replay(ex, pool, to_device(k_rows, w.shape.dtype, device),
               to_device(v_rows, w.shape.dtype, device))
    return ex, opool, pool


@pytest.mark.parametrize("make,P_k", [
    (lambda: wl.lognormal(256, batch=40), 16),
    (lambda: wl.lognormal(256, batch=40), 64),
    (lambda: wl.lognormal(64, batch=40), 32),
    (lambda: wl.batch32(num_blocks=8192), 16),      # P_a = 16: a view of one
])
def test_kernel_view_decode(pba, gpu, make, P_k):
    w = make()
    ex, opool, pool = _setup(w, gpu)
    P_a = w.shape.block_size
    say("kernel view", w.name, "P_a", P_a, "P_k", P_k)
    view = pool.kernel_view(P_k)
    split = view.split_log2
    q = to_device(wl.q_bits(w), w.shape.dtype, gpu)
    tab_a = torch.from_numpy(ex.tables).to(gpu)
    tab_k = pba.expand_block_tables(tab_a, split)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    for pt in (0, 512):
        out_a, lse_a = pba.paged_decode(pool, q, tab_a, lens, partition_tokens=pt)
        out_k, lse_k = pba.paged_decode(view, q, tab_k, lens, partition_tokens=pt)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_k) and torch.equal(lse_a, lse_k), pt
    ref, _ = att.paged_decode(opool, wl.q_bits(w), list(ex.tables), ex.seq_lens,
                              1 / math.sqrt(w.shape.head_dim))
    assert np.max(np.abs(out_k.cpu().numpy() - ref)) <= TOL


def test_kernel_view_f32(pba, gpu):
    """The fp32 path through a view: 32-row tiles read as 16-row blocks."""
    w = wl.Workload("f32_view", wl.Shape(32, 2, 1, 64, "f32", 40), 20261202 + 8100)
    w.actions = [("new",), ("prefill", 0, 150), ("new",), ("prefill", 1, 33), ("fork", 0),
                 ("prefill", 2, 20)]
    w.decode = [0, 1, 2]
    ex, opool, pool = _setup(w, gpu)
    say("f32 kernel view", w.shape)
    view = pool.kernel_view(16)
    q = to_device(wl.q_bits(w), "f32", gpu)
    tab_k = pba.expand_block_tables(torch.from_numpy(ex.tables).to(gpu), 1)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    out, _ = pba.paged_decode(view, q, tab_k, lens)
    torch.cuda.synchronize()
    ref, _ = att.paged_decode(opool, wl.q_bits(w), list(ex.tables), ex.seq_lens, 1 / math.sqrt(64))
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL


@pytest.mark.parametrize("make", [lambda: wl.lognormal(16, batch=64), wl.batch32,
                                  lambda: wl.lognormal(64, batch=48)])
def test_ragged_decode(pba, gpu, make):
    w = make()
    ex, opool, pool = _setup(w, gpu)
    P = w.shape.block_size
    entries, offsets = views.pack_ragged(ex.tables, ex.seq_lens, P)
    say("ragged", w.name, "entries", entries.size, "dense", ex.tables.size)
    q = to_device(wl.q_bits(w), w.shape.dtype, gpu)
    tab = torch.from_numpy(ex.tables).to(gpu)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    ent = torch.from_numpy(entries).to(gpu)
    off = torch.from_numpy(offsets).to(gpu)
    mb = ex.tables.shape[1]
    for pt in (0, 512):
        out_d, lse_d = pba.paged_decode(pool, q, tab, lens, partition_tokens=pt)
        out_r, lse_r = pba.paged_decode_ragged(pool, q, ent, off, lens, mb, partition_tokens=pt)
        torch.cuda.synchronize()
        assert torch.equal(out_d, out_r) and torch.equal(lse_d, lse_r), pt
    # Ragged over a kernel view: expand the compact entries, scale the offsets.
    if P >= 32:
        view = pool.kernel_view(P // 2)
        ent_k = pba.expand_block_tables(ent, 1)
        out_v, _ = pba.paged_decode_ragged(view, q, ent_k, off * 2, lens, mb * 2,
                                           partition_tokens=512)   # the plan of out_d
        torch.cuda.synchronize()
        assert torch.equal(out_v, out_d)
    ref, _ = att.paged_decode(opool, wl.q_bits(w), list(ex.tables), ex.seq_lens,
                              1 / math.sqrt(w.shape.head_dim))
    assert np.max(np.abs(out_r.cpu().numpy() - ref)) <= TOL


def test_ragged_validate_rejections(pba, gpu):
    w = wl.lognormal(16, batch=8)
    ex, opool, pool = _setup(w, gpu)
    entries, offsets = views.pack_ragged(ex.tables, ex.seq_lens, 16)
    q = to_device(wl.q_bits(w), "bf16", gpu)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    ent = torch.from_numpy(entries).to(gpu)
    mb = ex.tables.shape[1]
    say("ragged validate", w.shape)
    bad = offsets.copy()
    bad[3] = bad[2] - 1                                   # decreasing
    with pytest.raises(pba.PBAError) as e:
        pba.paged_decode_ragged(pool, q, ent, torch.from_numpy(bad).to(gpu), lens, mb)
    assert e.value.status == -6
    short = offsets.copy()
    short[1:] -= 1                                        # row 0 one entry short
    short[0] = 0
    with pytest.raises(pba.PBAError) as e:
        pba.paged_decode_ragged(pool, q, ent, torch.from_numpy(short).to(gpu), lens, mb)
    assert e.value.status == -6
    big = torch.tensor([1 << 30], dtype=torch.int32, device=gpu)
    with pytest.raises(pba.PBAError) as e:
        pba.expand_block_tables(big, 2)
    assert e.value.status == -6
