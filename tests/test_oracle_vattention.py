"""Pins for oracle.vattention: the pages' vAttention address algebra and
ledgers, the slot/page lifecycle (retention, reclamation, all-or-nothing
mapping), and decode over contiguous slot rows."""

import numpy as np
import pytest

from oracle import attention as att
from oracle import vattention as va
from oracle.bits import bits_to_f64
from oracle.pool import BitPool


def fixture_geometry(fx):
    return va.Geometry(fx["L"], fx["B"], fx["T_max"], fx["H_kv"], fx["d_h"], fx["b"], fx["G"])


def test_fixture_ledgers(golden):
    fx = golden("vattention.json")["fixture"]
    g = fixture_geometry(fx)
    e = fx["expect"]
    assert g.row_bytes == e["row_bytes"] and g.tokens_per_page == e["tokens_per_page"]
    assert g.slot_bytes == e["R"] and g.reserved_bytes == e["M_VA"]
    assert g.page_bundle_bytes == e["page_bundle"]
    a = va.Arena(g, fx["N_handle"])
    led = a.ledgers()
    assert led["phys_pool"] == e["M_phys_pool"] and led["va"] == e["M_VA"]
    assert led["mapped"] == 0 and led["free_handles"] == e["M_phys_pool"]


def test_checked_scalar(golden):
    fx = golden("vattention.json")
    g = fixture_geometry(fx["fixture"])
    s = fx["scalar"]
    A, u, q, delta = g.address(s["kind"], s["layer"], s["slot"], s["t"], s["h"], s["lane"])
    e = s["expect"]
    assert (u, q, delta, A) == (e["u"], e["q"], e["delta"], e["A_VA"])
    assert g.tensor_base("V", 1) == e["base"]


def test_addresses_are_a_bijection_onto_the_reservation(golden):
    """Every scalar of every tensor, slot and row of the fixture has its own
    address, all inside [0, M_VA); a slot's rows stay in its subrange, and a
    row's page is the floor of its offset."""
    g = fixture_geometry(golden("vattention.json")["fixture"])
    seen = set()
    for kind in "KV":
        for layer in range(g.layers):
            for slot in range(g.slots):
                lo = g.tensor_base(kind, layer) + slot * g.slot_bytes
                for t in range(g.max_tokens):
                    for h in range(g.kv_heads):
                        for d in range(g.head_dim):
                            A, u, q, delta = g.address(kind, layer, slot, t, h, d)
                            assert lo <= A < lo + g.slot_bytes and q * g.page_bytes + delta == u
                            assert q < g.pages_for(t + 1)
                            for byte in range(g.scalar_bytes):
                                seen.add(A + byte)
    assert len(seen) == g.reserved_bytes and min(seen) == 0 and max(seen) == g.reserved_bytes - 1


def test_page_group_staircase(golden):
    fx = golden("vattention.json")["staircase"]
    for G, tpp, n0, w0, n1, w1 in zip(fx["page_bytes"], fx["tokens_per_page"], fx["T1024"]["groups"],
                                      fx["T1024"]["waste"], fx["T1025"]["groups"], fx["T1025"]["waste"]):
        assert G // fx["row_bytes"] == tpp
        assert va.page_group_staircase(1024, fx["row_bytes"], G) == (n0, w0)
        assert va.page_group_staircase(1025, fx["row_bytes"], G) == (n1, w1)


def test_delayed_reclamation_reuses_capacity_not_rows(golden):
    g = fixture_geometry(golden("vattention.json")["fixture"])
    a = va.Arena(g, 12)
    gen_a = a.allocate(0)
    assert a.ensure(0, 8) == 2                     # A maps slot 0 pages [0, 1]
    a.commit(0, 8)
    a.free(0, retain=True)                         # A completes: pages stay mapped
    assert a.slots[0].mapped_pages == 2 and a.ledgers()["inactive_retained"] == 2 * 256
    gen_c = a.allocate(0)                          # C receives slot 0
    assert gen_c == gen_a + 1 and a.slots[0].valid_tokens == 0
    assert a.ensure(0, 3) == 0                     # needs only page 0: no new mapping
    assert a.maps == 2 and a.unmaps == 0
    a.check()


def test_growth_reclaims_an_inactive_bundle(golden):
    """D grows from 8 to 9 tokens with no free handle: B's inactive bundle is
    unmapped and becomes D's page q = 2 (0x06F); one more page fails and
    changes nothing."""
    g = fixture_geometry(golden("vattention.json")["fixture"])
    a = va.Arena(g, 12)
    B, D = 1, 2
    a.allocate(B)
    a.ensure(B, 4)
    a.commit(B, 4)
    b_handles = list(a.mapping[(B, 0)])
    a.free(B, retain=True)
    a.allocate(D)
    assert a.ensure(D, 8) == 2 and a.ledgers()["free_handles"] == 0
    a.commit(D, 8)
    assert a.ensure(D, 9) == 1
    assert a.mapping[(D, 2)] == b_handles and a.slots[B].mapped_pages == 0
    assert a.unmaps == 1
    a.commit(D, 9)
    a.check()
    before = (list(a.free_handles), dict(a.mapping), [s.mapped_pages for s in a.slots])
    a.allocate(0)
    with pytest.raises(va.MappingFailure):
        a.ensure(0, 1)
    assert (list(a.free_handles), dict(a.mapping), [s.mapped_pages for s in a.slots]) == before
    with pytest.raises(ValueError):
        a.commit(0, 1)                             # rows beyond the frontier


@pytest.mark.parametrize("seed", range(5))
def test_random_lifecycles_reconcile(seed):
    rng = np.random.default_rng(70 + seed)
    g = va.Geometry(2, 5, 40, 2, 4, 2, 64)
    a = va.Arena(g, int(rng.integers(8, 40)))
    for _ in range(300):
        s = int(rng.integers(g.slots))
        slot = a.slots[s]
        op = rng.integers(3)
        if not slot.active:
            a.allocate(s)
        elif op == 0:
            a.free(s, retain=bool(rng.integers(2)))
        else:
            want = min(g.max_tokens, slot.valid_tokens + int(rng.integers(1, 12)))
            state = (list(a.free_handles), dict(a.mapping), [x.mapped_pages for x in a.slots])
            try:
                a.ensure(s, want)
                a.commit(s, want)
                assert a.capacity(s) >= want
            except va.MappingFailure:
                assert state == (list(a.free_handles), dict(a.mapping),
                                 [x.mapped_pages for x in a.slots])
        a.check()


def test_contiguous_decode_equals_paged_decode():
    """The slot-indexed decode (no block table) equals the pinned paged decode
    when the same rows sit in a paged pool behind a table."""
    rng = np.random.default_rng(3)
    S, Tm, H, d, G, P = 4, 50, 2, 16, 3, 16
    k = rng.integers(0, 1 << 16, size=(S, Tm, H, d), dtype=np.uint16) & np.uint16(0xBFFF)
    v = rng.integers(0, 1 << 16, size=(S, Tm, H, d), dtype=np.uint16) & np.uint16(0xBFFF)
    kf, vf = bits_to_f64(k, "bf16"), bits_to_f64(v, "bf16")
    slot_index = [2, 0, 3, 2]
    lens = [50, 17, 1, 33]
    q = rng.integers(0, 1 << 16, size=(4, H * G, d), dtype=np.uint16) & np.uint16(0xBFFF)
    out, lse = va.contiguous_decode(kf, vf, bits_to_f64(q, "bf16"), slot_index, lens, 0.25, G)
    nb = S * 4
    kp = np.zeros((nb, H, P, d), np.uint16)
    vp = np.zeros((nb, H, d, P), np.uint16)
    for s in range(S):
        for t in range(Tm):
            b, o = s * 4 + t // P, t % P
            kp[b, :, o] = k[s, t]
            vp[b, :, :, o] = v[s, t]
    tables = [[s * 4 + j for j in range(4)] for s in slot_index]
    ref, ref_lse = att.paged_decode(BitPool(kp, vp, "bf16"), q, tables, lens, 0.25)
    assert np.max(np.abs(out - ref)) <= 1e-15 and np.max(np.abs(lse - ref_lse)) <= 1e-13
