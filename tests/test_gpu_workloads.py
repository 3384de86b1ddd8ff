"""GPU parity at the workload sizes: batch32, shared prefix with copy-on-write,
lognormal lengths at P in {16, 64, 256}, and the long-context workloads at full
size in the launch configuration bench.py times (sampled output rows)."""
import pytest

import workloads as wl
from test_gpu_parity import pba, run_workload  # noqa: F401  (fixture + helper)

pytestmark = pytest.mark.gpu


def test_batch32(pba, gpu):
    run_workload(pba, wl.batch32(), gpu)


def test_shared_prefix_with_cow(pba, gpu):
    w = wl.shared_prefix()
    ex, pool, out, lse = run_workload(pba, w, gpu)
    n_copies = sum(len(op[1]) for op in ex.ops if op[0] == "copy")
    # One copy per sibling whose shared tail was partial (suffix mod 16 != 0).
    suffix = [a[2] for a in w.actions if a[0] == "prefill" and a[1] != 0]
    assert n_copies == sum(1 for s in suffix if (2000 + s) % 16 != 0)
    # Shared prefix blocks: refcount = children + siblings that still map them.
    first = ex.alloc.table(1)[0]
    assert ex.alloc.ref[first] == 128


@pytest.mark.parametrize("P", [16, 64, 256])
def test_lognormal_block_sizes(pba, gpu, P):
    run_workload(pba, wl.lognormal(P), gpu)


def test_long16k_sampled(pba, gpu):
    w = wl.long16k()
    pairs = [(0, 0), (3, 5), (7, 7)]
    run_workload(pba, w, gpu, pairs=pairs)


def test_long64k_sampled(pba, gpu):
    w = wl.long64k()
    run_workload(pba, w, gpu, pairs=[(0, 2), (0, 6)])


