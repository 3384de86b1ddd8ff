"""GPU tests of the binding's workspace handling (the cached, zero-filled
workspace the decode calls use when the caller passes none).

* Two decode layouts whose workspaces have the same byte size but different
  counter regions get separate buffers: the second call's completion counters
  must not sit on the first call's partial states.
* A decode on an explicit stream that is not torch's current stream gets a
  workspace zeroed on that stream, so the fill is ordered before the launch.
Every case prints its name and shapes (flushed) before its GPU work.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from harness import execute, gpu_pool, gpu_replay, oracle_pool, to_device
from oracle import attention as att
from test_gpu_parity import TOL, pba, run_workload, say, small_workload  # noqa: F401

pytestmark = pytest.mark.gpu


def test_workspace_cache_distinguishes_equal_size_layouts(pba, gpu):
    """6 rows at 90 partitions and 268 rows at 2 partitions (8 kv heads, G = 1,
    d = 64) need 1,140,736 workspace bytes each, but the second layout's
    counters cover the first one's (m, l) states."""
    rng = np.random.default_rng(2026)
    lens_a = [int(x) for x in rng.integers(300, 601, size=6)]
    lens_b = [int(x) for x in rng.integers(257, 513, size=268)]
    wa = small_workload("bf16", 16, 64, 8, 1, lens_a, 20261202 + 3100)
    wb = small_workload("bf16", 16, 64, 8, 1, lens_b, 20261202 + 3200)
    say("workspace layouts", wa.shape, wb.shape)
    pool_a = pba.KVPool.empty(8, 16, 8, 64, torch.bfloat16, gpu)
    need_a = pba.paged_decode_workspace_bytes(pool_a, 8, 6, 1440, 256)
    need_b = pba.paged_decode_workspace_bytes(pool_a, 8, 268, 32, 256)
    assert need_a == need_b == 1140736
    assert pba.paged_decode_plan(pool_a, 8, 6, 1440, 256) == (256, 90)
    assert pba.paged_decode_plan(pool_a, 8, 268, 32, 256) == (256, 2)
    pba._WORKSPACES.clear()
    run_workload(pba, wa, gpu, max_blocks=1440, check_pool=False, partition_tokens=256)
    run_workload(pba, wb, gpu, max_blocks=32, check_pool=False, partition_tokens=256)
    run_workload(pba, wa, gpu, max_blocks=1440, check_pool=False, partition_tokens=256)
    layouts = sorted(k[2] for k in pba._WORKSPACES)
    assert len(layouts) == 2 and layouts[0] != layouts[1]
    torch.cuda.synchronize()
    for key, ws in pba._WORKSPACES.items():
        _, batch, kv_heads = key[2][:3]
        counters = ws[:4 * batch * kv_heads].view(torch.int32)
        assert int(counters.abs().sum()) == 0, f"counters left nonzero for {key[2]}"


def test_explicit_stream_without_context(pba, gpu):
    """stream=s with s not current: the cached workspace is allocated and
    zeroed on s, and the result matches the oracle."""
    w = small_workload("bf16", 32, 128, 2, 4, [100, 700, 1500, 2049], 20261202 + 3300)
    say("explicit stream", w.shape)
    ex = execute(w)
    k_rows, v_rows = wl.kv_rows(w, ex.n_writes)
    opool = oracle_pool(ex, k_rows, v_rows)
    pool = gpu_pool(ex, gpu)
    gpu_replay(ex, pool, to_device(k_rows, "bf16", gpu), to_device(v_rows, "bf16", gpu))
    qb = wl.q_bits(w)
    q = to_device(qb, "bf16", gpu)
    tables = torch.from_numpy(ex.tables).to(gpu)
    lens = torch.from_numpy(ex.seq_lens).to(gpu)
    scale = 1.0 / math.sqrt(w.shape.head_dim)
    pba._WORKSPACES.clear()
    s = torch.cuda.Stream(device=gpu)
    s.wait_stream(torch.cuda.current_stream(gpu))
    out, lse = pba.paged_decode(pool, q, tables, lens, scale, partition_tokens=256, stream=s)
    s.synchronize()
    (key,) = list(pba._WORKSPACES)
    assert key[1] == s.cuda_stream
    ref, ref_lse = att.paged_decode(opool, qb, list(ex.tables), ex.seq_lens, scale)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    say("explicit stream max abs err", err, "lse err", lerr)
    assert err <= TOL and lerr <= TOL
