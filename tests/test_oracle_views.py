"""Pins of oracle/views.py (kernel views of allocator pools, ragged tables).

* The pages' expansion example ("M5.3", 0x0AC): P_a = 32, P_k = 16 turns
  allocator ids [3, 7] into kernel ids [6, 7, 14, 15]; P_a = 64, P_k = 16 gives
  four kernel ids per allocator id; a kernel block larger than the allocator
  block is rejected.
* Reading a request through the expanded table with the split rule returns
  exactly the rows of the allocator-table gather (random pools, every q).
* The compact table of the pages' lengths [64, 63, 17, 1] at P_k = 16 (0x0AB):
  n_r = [4, 4, 2, 1], offsets [0, 4, 8, 10, 11], 11 used cells against 16
  dense; unpacking returns each row's first n_r entries.
"""
import numpy as np
import pytest

from oracle import views
from oracle.pool import BitPool
import workloads as wl


def test_page_expansion_examples():
    assert views.expand_table([3, 7], 32, 16) == [6, 7, 14, 15]
    assert views.expand_table([5], 64, 16) == [20, 21, 22, 23]
    assert views.expand_table([0, 1], 16, 16) == [0, 1]
    with pytest.raises(ValueError):
        views.expand_table([1], 16, 32)
    with pytest.raises(ValueError):
        views.expand_table([1], 48, 32)


@pytest.mark.parametrize("P_a,P_k,dtype", [(32, 16, "bf16"), (64, 16, "f32"), (256, 64, "bf16"),
                                           (256, 16, "bf16"), (64, 64, "bf16")])
def test_split_gather_equals_allocator_gather(P_a, P_k, dtype):
    rng = np.random.default_rng(P_a * 1000 + P_k)
    nb, H, d = 12, 2, 64
    k = wl.normal_bits(int(rng.integers(1 << 30)), (nb, H, P_a, d), dtype)
    v = wl.normal_bits(int(rng.integers(1 << 30)), (nb, H, d, P_a), dtype)
    pool = BitPool(k, v, dtype)
    for _ in range(5):
        T = int(rng.integers(1, 5 * P_a))
        n_a = -(-T // P_a)
        table = [int(x) for x in rng.choice(nb, size=n_a, replace=False)]
        ktab = views.expand_table(table, P_a, P_k)
        for h in range(H):
            K0, V0 = pool.gather(table, T, h)
            K1, V1 = views.gather_kernel_view(pool, ktab, T, h, P_k)
            assert np.array_equal(K0, K1) and np.array_equal(V0, V1)


def test_page_ragged_fixture():
    lens = [64, 63, 17, 1]
    dense = np.arange(100, 116, dtype=np.int32).reshape(4, 4)
    entries, offsets = views.pack_ragged(dense, lens, 16)
    assert offsets.tolist() == [0, 4, 8, 10, 11]
    assert entries.size == 11 and dense.size == 16
    for r, T in enumerate(lens):
        assert views.unpack_ragged(entries, offsets, r).tolist() == dense[r, :-(-T // 16)].tolist()
