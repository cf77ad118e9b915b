"""CPU checks of the test harness's oracle half (what the GPU tests compare against)."""

import numpy as np
import pytest

import paged_kv_cache_117_amd as pa
from harness import Step, oracle_step
from workloads import make_custom, make_workload


@pytest.mark.parametrize("key", ["c1", "c4b"])
def test_oracle_step_runs_and_is_finite(key):
    w = make_workload(key)
    rows = [0, 1, 2, 3] if key == "c1" else [0, 7, 8]
    st, k, v, out = oracle_step(w, rows=rows)
    assert out.shape == (len(rows), w.num_q_heads, w.head_dim)
    assert np.all(np.isfinite(out))
    st2, _, _, none = oracle_step(w, rows=[])
    assert none.shape[0] == 0


def test_poison_keeps_exactly_the_cached_positions():
    w = make_custom("p", "fp32", [1, 5, 16, 17, 33], 2, 2, 64, seed=3, num_blocks=12)
    st = Step(w, lambda n, bs, o: pa.BlockManager(n, bs, o))
    kept = np.isfinite(st.k0[:, 0, :, 0])
    assert kept.sum() == int((w.context_lens - 1).sum())
    # the slot the step writes is poisoned
    for slot in st.slots:
        assert not kept[slot // 16, slot % 16]


def test_bench_kv_utilization_counts_shared_blocks_once():
    """The bench's utilisation figure: filled slots over slots of blocks in
    use, a shared block counted once.  Sequence 0 has 20 tokens (blocks
    A: 16, B: 4); its fork shares A and B, then appends 1 token, which copies
    B (count 2) into C and writes there (5 filled).  In use: A, B, C of 8."""
    import os
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    bm = pa.BlockManager(8, 16)
    bm.add_seq(0)
    bm.append(0, 20)
    bm.fork(0, 1)
    bm.append(1, 1)
    bm.take_copies()
    tables = bm.tables([0, 1], 4)
    u = bench.kv_utilization(bm, [0, 1], tables, 16, 8)
    assert u["kv_blocks_in_use_frac"] == 3 / 8
    assert u["kv_slot_utilization"] == round((16 + 4 + 5) / 48, 4)


def test_roofline_bound_follows_the_ridge_point():
    """The prefill record's bound is the larger lower bound on time: flops at
    2,500 TFLOP/s or bytes at 8,000 GB/s (ridge 312.5 flops per byte).  A
    matrix-heavy launch (1,000 flops per byte) reports TFLOP/s against the
    matrix peak, one below the ridge (100 flops per byte) GB/s against HBM,
    and both fractions come out of the same time."""
    import os
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    # 1e12 flops over 1e9 bytes in 1 ms: 1,000 TFLOP/s and 1,000 GB/s
    r = bench.roofline_bound(1e12, 1e9, 1.0, 2500.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == 1000.0 and r["frac"] == 0.4
    assert r["mfma_frac"] == 0.4 and r["hbm_frac"] == 0.125
    assert r["arithmetic_intensity"] == 1000.0 and r["ridge"] == 312.5
    # 1e11 flops over 1e9 bytes in 0.25 ms: 400 TFLOP/s and 4,000 GB/s
    r = bench.roofline_bound(1e11, 1e9, 0.25, 2500.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == 4000.0 and r["frac"] == 0.5
    assert r["mfma_frac"] == 0.16 and r["hbm_frac"] == 0.5
    # exactly at the ridge the matrix bound is taken
    assert bench.roofline_bound(312.5e9, 1e9, 1.0, 2500.0)["bound"] == "mfma"
