"""GPU tests of the contiguous virtual K/V arena (pba_vkv_*) and the
slot-indexed decode (pba_paged_decode_contiguous), through the C ABI.

Every test runs in validate mode: the library checks each append and decode
against the slots' mapped frontiers before launching, so no kernel can touch
an unmapped page.

* Ledgers: a script of map / free operations leaves the arena's mapped,
  retained, free and pool bytes, its bundle map / unmap counts and every
  slot's capacity equal to the oracle's lifecycle model after every step
  (including reclamation and a refused request that changes nothing).
* Parity: rows appended through the arena (as a cache group, every layer in
  one launch) decode by slot index within 2e-3 of the oracle's slot-indexed
  decode, and bitwise equal to the paged decode of the same memory through a
  block table, and to the same decode on an ordinary device buffer.
* Reuse: a slot freed with its pages retained serves a new request that
  writes its own rows; reclamation moves pages from an inactive slot to a
  growing one without disturbing other slots.
* Residency: a 32 GiB reservation costs no device memory until pages map.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from harness import to_device
from oracle import vattention as va
from oracle.bits import bits_to_f64

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


def _ledgers_match(arena, model, slots):
    led = arena.ledgers()
    o = model.ledgers()
    assert led["mapped_bytes"] == o["mapped"]
    assert led["inactive_retained_bytes"] == o["inactive_retained"]
    assert led["free_bytes"] == o["free_handles"]
    assert led["pool_bytes"] == o["phys_pool"]
    assert led["reserved_bytes"] == o["va"]
    assert (led["bundle_maps"], led["bundle_unmaps"]) == (model.maps, model.unmaps)
    for s in range(slots):
        assert arena.capacity(s) == model.capacity(s)


def test_lifecycle_ledgers_match_oracle(pba, gpu):
    L, B, Tm, H, d, P, G = 2, 4, 300, 2, 128, 16, 65536
    handles = 2 * L * 6                       # six page bundles in the pool
    say("arena lifecycle", (L, B, Tm, H, d, P, G), "handles", handles)
    arena = pba.VKVArena(L, B, Tm, H, d, P, G, num_handles=handles)
    model = va.Arena(va.Geometry(L, B, Tm, H, d, 2, G), handles)
    rng = np.random.default_rng(11)
    refused = 0
    for step in range(80):
        s = int(rng.integers(B))
        if model.slots[s].active and rng.random() < 0.3:
            retain = bool(rng.integers(2))
            model.free(s, retain)
            arena.free(s, retain)
        else:
            want = int(rng.integers(1, Tm + 1))
            was_active = model.slots[s].active
            state = (list(model.free_handles), dict(model.mapping),
                     [x.mapped_pages for x in model.slots], [x.active for x in model.slots])
            if not was_active:
                model.allocate(s)
            try:
                model.ensure(s, want)
            except va.MappingFailure:
                if not was_active:            # the library leaves the slot as it was
                    model.slots[s].active = False
                    model.slots[s].generation -= 1
                assert state[:3] == (list(model.free_handles), dict(model.mapping),
                                     [x.mapped_pages for x in model.slots])
                with pytest.raises(pba.PBAError) as e:
                    arena.map(s, want)
                assert e.value.status == -10
                refused += 1
            else:
                arena.map(s, want)
        _ledgers_match(arena, model, B)
        model.check()
    say("   maps", model.maps, "unmaps", model.unmaps, "refused", refused)
    assert model.unmaps > 0 and refused > 0   # the script exercised reclamation and refusal
    arena.close()


def _write_slot(pba, arena, slot, t0, k, v, gpu):
    """Rows t0 .. t0+n-1 of every layer: k, v bits [n, L, H, d]."""
    n = k.shape[0]
    ids = torch.from_numpy(arena.slot_ids(slot, np.arange(t0, t0 + n, dtype=np.int64))).to(gpu)
    pba.kv_append_bundle([arena], [ids], [to_device(k, "bf16", gpu)], [to_device(v, "bf16", gpu)])


@pytest.mark.parametrize("P,d,G", [(16, 128, 65536), (64, 64, 2 << 20), (32, 128, 1 << 20)])
def test_contiguous_decode_parity(pba, gpu, P, d, G):
    L, B, H, Hq = 2, 5, 2, 8
    Tm = 700
    say("contiguous decode", dict(P=P, d=d, G=G))
    arena = pba.VKVArena(L, B, Tm, H, d, P, G)
    lens = np.array([1, 700, 333, 64, 517], dtype=np.int32)
    seed = wl.seed_for("bundle", 50 + P)
    rows = {}
    for s, T in enumerate(lens):
        arena.map(s, int(T))
        k = wl.normal_bits(seed + 2 * s, (int(T), L, H, d), "bf16")
        v = wl.normal_bits(seed + 2 * s + 1, (int(T), L, H, d), "bf16")
        cut = int(T) // 3                  # two appends per slot
        _write_slot(pba, arena, s, 0, k[:cut], v[:cut], gpu)
        _write_slot(pba, arena, s, cut, k[cut:], v[cut:], gpu)
        rows[s] = (k, v)
    order = np.array([3, 1, 4, 0, 2, 1], dtype=np.int32)   # batch rows -> slots (one slot twice)
    T_b = lens[order]
    q_bits = wl.normal_bits(seed + 99, (L, len(order), Hq, d), "bf16")
    slot_index = torch.from_numpy(order).to(gpu)
    seq = torch.from_numpy(T_b).to(gpu)
    bps = arena.blocks_per_slot
    tab = (order[:, None] * bps + np.arange(bps)[None, :]).astype(np.int32)
    tab[np.arange(bps)[None, :] >= -(-T_b[:, None] // P)] = -1   # entries past each row's blocks
    tables = torch.from_numpy(tab).to(gpu)
    scale = 1 / math.sqrt(d)
    for layer in range(L):
        pool = arena.layer(layer)
        q = to_device(q_bits[layer], "bf16", gpu)
        for pt in (0, 256):
            out_c, lse_c = pba.paged_decode_contiguous(pool, q, slot_index, bps, seq, scale,
                                                       partition_tokens=pt)
            out_p, lse_p = pba.paged_decode(pool, q, tables, seq, scale, partition_tokens=pt)
            torch.cuda.synchronize()
            assert torch.equal(out_c, out_p) and torch.equal(lse_c, lse_p), (layer, pt)
        rk = [bits_to_f64(rows[s][0][:, layer], "bf16") if s in rows else None for s in range(B)]
        rv = [bits_to_f64(rows[s][1][:, layer], "bf16") if s in rows else None for s in range(B)]
        ref, ref_lse = va.contiguous_decode(rk, rv, bits_to_f64(q_bits[layer], "bf16"), order,
                                            T_b, scale, Hq // H)
        err = np.max(np.abs(out_c.cpu().numpy() - ref))
        say("   layer", layer, "max err", err)
        assert err <= TOL and np.max(np.abs(lse_c.cpu().numpy() - ref_lse)) <= TOL
        # The same decode over an ordinary device buffer laid out like the arena.
        if layer == 0:
            nb = arena.num_blocks
            kbuf = torch.zeros((nb, H, P, d), dtype=torch.bfloat16, device=gpu)
            vbuf = torch.zeros((nb, H, d, P), dtype=torch.bfloat16, device=gpu)
            plain = pba.KVPool(kbuf, vbuf)
            for s, T in enumerate(lens):
                ids = torch.from_numpy(arena.slot_ids(s, np.arange(T, dtype=np.int64))).to(gpu)
                pba.kv_append(plain, ids, to_device(rows[s][0][:, 0], "bf16", gpu),
                              to_device(rows[s][1][:, 0], "bf16", gpu))
            out_b, _ = pba.paged_decode_contiguous(plain, q, slot_index, bps, seq, scale)
            out_c0, _ = pba.paged_decode_contiguous(pool, q, slot_index, bps, seq, scale)
            torch.cuda.synchronize()
            assert torch.equal(out_b, out_c0)
    arena.close()


def test_retained_slot_and_reclamation(pba, gpu):
    L, B, H, d, P, G = 1, 3, 2, 128, 16, 65536     # 128 tokens per page
    Hq = 4
    arena = pba.VKVArena(L, B, 512, H, d, P, G, num_handles=2 * L * 5)
    say("retention and reclamation")
    seed = wl.seed_for("bundle", 80)

    def rows(s, T, salt):
        return (wl.normal_bits(seed + 10 * salt + s, (T, L, H, d), "bf16"),
                wl.normal_bits(seed + 10 * salt + s + 5, (T, L, H, d), "bf16"))

    def check(order, lens, data):
        q_bits = wl.normal_bits(seed + 77, (len(order), Hq, d), "bf16")
        out, _ = pba.paged_decode_contiguous(arena.layer(0), to_device(q_bits, "bf16", gpu),
                                             torch.tensor(order, dtype=torch.int32, device=gpu),
                                             arena.blocks_per_slot,
                                             torch.tensor(lens, dtype=torch.int32, device=gpu))
        torch.cuda.synchronize()
        rk = [bits_to_f64(data[s][0][:, 0], "bf16") if s in data else None for s in range(B)]
        rv = [bits_to_f64(data[s][1][:, 0], "bf16") if s in data else None for s in range(B)]
        ref, _ = va.contiguous_decode(rk, rv, bits_to_f64(q_bits, "bf16"), order, lens,
                                      1 / math.sqrt(d), Hq // H)
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL

    data = {}
    arena.map(0, 300)                               # 3 pages
    data[0] = rows(0, 300, 1)
    _write_slot(pba, arena, 0, 0, *data[0], gpu)
    arena.map(1, 200)                               # 2 pages: pool exhausted
    data[1] = rows(1, 200, 1)
    _write_slot(pba, arena, 1, 0, *data[1], gpu)
    check([0, 1], [300, 200], data)
    arena.free(0, retain=True)                      # request of slot 0 ends, pages kept
    maps = arena.ledgers()["bundle_maps"]
    arena.map(0, 100)                               # new request on slot 0: capacity reused
    assert arena.ledgers()["bundle_maps"] == maps
    data[0] = rows(0, 100, 2)                       # it writes its own rows
    _write_slot(pba, arena, 0, 0, *data[0], gpu)
    check([0, 1], [100, 200], data)
    arena.free(0, retain=True)
    arena.map(2, 256)                               # takes slot 0's two highest pages
    led = arena.ledgers()
    assert led["bundle_unmaps"] == 2 and arena.capacity(0) == 128 and arena.capacity(2) == 256
    data[2] = rows(2, 256, 3)
    _write_slot(pba, arena, 2, 0, *data[2], gpu)
    check([2, 1], [256, 200], data)                 # slot 1 undisturbed
    with pytest.raises(pba.PBAError) as e:          # 2 more pages than the pool can give
        arena.map(1, 512)
    assert e.value.status == -10 and arena.capacity(1) == 256
    # Frontier checks in validate mode: past-capacity decode and append refused.
    with pytest.raises(pba.PBAError) as e:
        check([2], [257], data)
    assert e.value.status == -6
    ids = torch.tensor([arena.slot_ids(2, 256)], dtype=torch.int64, device=gpu)
    one = torch.zeros((1, L, H, d), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(pba.PBAError) as e:
        pba.kv_append_bundle([arena], [ids], [one], [one])
    assert e.value.status == -6
    arena.free(2, retain=False)
    assert arena.capacity(2) == 0
    arena.close()


def test_reservation_is_not_residency(pba, gpu):
    """32 GiB of virtual reservation; device memory drops only by mapped pages."""
    L, B, H, d, P, G = 4, 64, 8, 128, 16, 2 << 20
    Tm = 32768                                      # 64 MiB per slot-tensor, 8 tensors, 64 slots
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    arena = pba.VKVArena(L, B, Tm, H, d, P, G)
    led = arena.ledgers()
    say("reservation", led["reserved_bytes"] >> 30, "GiB")
    assert led["reserved_bytes"] == 2 * L * B * 64 * (1 << 20)
    free1, _ = torch.cuda.mem_get_info()
    arena.map(0, 3000)                              # 3 pages x 8 tensors = 48 MiB
    free2, _ = torch.cuda.mem_get_info()
    assert led["mapped_bytes"] == 0 and arena.ledgers()["mapped_bytes"] == 3 * 8 * G
    assert free0 - free1 < (256 << 20)
    assert free1 - free2 >= 3 * 8 * G - (4 << 20)
    arena.close()
