"""Seeded random shapes through the fused decode step (pba_paged_decode_append)
against the separate calls and the binary64 oracle.

Each case draws its block size (16-256), head_dim (64, 128), kv heads (1-8),
G (1-16), pool dtype (bf16, sometimes fp32), batch (1-24), lengths (1-1500,
log-uniform), which rows append, and the decomposition (library plan, 256 or
512-token partitions, balanced), then runs tests/test_gpu_fused's check: pools
bit for bit against the oracle and against kv_append + paged_decode, out and
lse bit for bit between the two, and within 2e-3 of the oracle.  The draws
come from a fixed seed per case, printed before the case runs."""
import numpy as np
import pytest

from test_gpu_fused import run_fused, step_workload
from test_gpu_parity import pba, say  # noqa: F401

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw(case):
    rng = np.random.default_rng(20261202 + 7700 + case)
    P = int(rng.choice([16, 32, 64, 128, 256]))
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    B = int(rng.integers(1, 25))
    lengths = [int(x) for x in np.exp(rng.uniform(0, np.log(1500), size=B)).astype(int) + 1]
    appends = [int(rng.random() < 0.7) for _ in range(B)]
    appends[0] = 1
    part = int(rng.choice([0, 256, 512, -1]))
    return P, d, Hkv, G, dtype, lengths, appends, part


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_fused_step(pba, gpu, case):
    P, d, Hkv, G, dtype, lengths, appends, part = draw(case)
    say("random case", case, "P", P, "d", d, "Hkv", Hkv, "G", G, dtype, "B", len(lengths),
        "partition", part)
    w = step_workload(dtype, P, d, Hkv, G, lengths, appends, 20261202 + 7700 + case)
    run_fused(pba, w, gpu, appends, part)
