"""GPU: the Python example in README.md runs as written, and both of its
outputs (the prefill of two prompts, then one decode step) match the oracle."""

import os
import re

import numpy as np
import pytest

import oracle
from harness import TOL, to_host_storage

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _example_code():
    blocks = re.findall(r"```python\n(.*?)```", open(README).read(), flags=re.S)
    assert blocks, "README.md holds no python example"
    return blocks[0]


def test_readme_example_runs_and_matches_the_oracle():
    import torch

    print("case README example", flush=True)
    ns = {}
    exec(compile(_example_code(), README, "exec"), ns)
    torch.cuda.synchronize()
    D = ns["D"]
    scale = float(np.float32(D ** -0.5))
    k = to_host_storage(ns["k_pool"], "bf16")
    v = to_host_storage(ns["v_pool"], "bf16")
    tables = ns["tables"].cpu().numpy()

    # the prefill rows: positions below each prompt's length, which the decode
    # step's writes (at positions 300 and 37) do not touch
    want = oracle.prefill(to_host_storage(ns["q"], "bf16"), k, v, tables, [300, 37], [0, 300, 337], scale, "bf16")
    got = oracle.storage_to_f64(to_host_storage(ns["out"], "bf16"), "bf16")
    assert np.isfinite(got).all()
    assert np.abs(got - want).max() <= TOL["bf16"]

    # the decode step, with its new tokens in the pools
    want1 = oracle.decode(to_host_storage(ns["q1"], "bf16"), k, v, tables, [301, 38], scale, "bf16")
    got1 = oracle.storage_to_f64(to_host_storage(ns["out1"], "bf16"), "bf16")
    assert np.isfinite(got1).all()
    assert np.abs(got1 - want1).max() <= TOL["bf16"]
    # and the new tokens sit where the block tables put them
    for s, pos in ((0, 300), (1, 37)):
        blk, off = int(tables[s][pos // 16]), pos % 16
        assert np.array_equal(k[blk, :, off], to_host_storage(ns["k1"], "bf16")[s])
        assert np.array_equal(v[blk, :, off], to_host_storage(ns["v1"], "bf16")[s])
