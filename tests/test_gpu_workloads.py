"""GPU parity at the workload sizes: batch32, shared prefix with copy-on-write,
lognormal lengths at P in {16, 64, 256}, and the long-context workloads at full
size in the launch configuration bench.py times.  Every (request, kv head)
pair of every workload is compared with the binary64 oracle (out and lse),
and the whole pool bit for bit."""
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


def test_long16k_all_pairs(pba, gpu):
    """8 x 16,384 tokens, 4 partitions of 4096 per (request, kv head), merged
    in the launch: all 64 pairs against the oracle."""
    run_workload(pba, wl.long16k(), gpu)


def test_long64k_all_pairs(pba, gpu):
    """1 x 65,536 tokens, 32 partitions of 2048 per kv head: all 8 kv heads."""
    run_workload(pba, wl.long64k(), gpu)


