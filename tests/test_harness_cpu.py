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
