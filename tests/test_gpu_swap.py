"""GPU parity of pa_swap_blocks: preemption by swapping blocks to pinned host
memory and back, bit for bit against the oracle, and attention unchanged
after the round trip."""

import numpy as np
import pytest

import oracle
from harness import GpuStep, to_f64, to_host_storage
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype.itemsize == 2 else a.view(np.uint32)


def _pinned_like(t, n_blocks, fill):
    import torch

    h = torch.empty((n_blocks,) + tuple(t.shape[1:]), dtype=t.dtype, pin_memory=True)
    h.fill_(fill)
    return h


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("fp16", 8, 2, 64), ("fp32", 4, 4, 64)])
@pytest.mark.parametrize("pairs_on_host", [False, True])
def test_swap_out_and_in_round_trip(dtype, hq, hkv, d, pairs_on_host):
    import torch

    import paged_kv_cache_117_amd as pa

    w = make_custom(f"sw_{dtype}", dtype, [37, 300, 16, 129, 64, 250], hq, hkv, d, seed=41)
    print(f"case swap {dtype} pairs_on_host={pairs_on_host}", flush=True)
    g = GpuStep(w)
    out_before = g.run().clone()
    torch.cuda.synchronize()
    k_dev0 = to_host_storage(g.k, dtype)
    v_dev0 = to_host_storage(g.v, dtype)
    tables = g.st.tables.copy()
    victims = [1, 3, 5]  # preempted sequences
    blocks = []
    for s in victims:
        nb = -(-int(w.context_lens[s]) // 16)
        blocks += [int(b) for b in tables[s, :nb]]
    n_host = len(blocks) + 3
    hk = _pinned_like(g.k, n_host, float("nan"))
    hv = _pinned_like(g.v, n_host, float("nan"))
    host_slot = np.random.default_rng(1).permutation(n_host)[:len(blocks)]
    out_pairs = np.stack([blocks, host_slot], axis=1).astype(np.int32)
    pt = torch.from_numpy(out_pairs)
    pt = pt.pin_memory() if pairs_on_host else pt.cuda()
    pa.swap_blocks(hk, hv, g.k, g.v, pt)
    torch.cuda.synchronize()
    want_hk, want_hv = oracle.swap_blocks(to_host_storage(_pinned_like(g.k, n_host, float("nan")), dtype),
                                          to_host_storage(_pinned_like(g.v, n_host, float("nan")), dtype),
                                          k_dev0, v_dev0, out_pairs)
    assert np.array_equal(_bits(to_host_storage(hk, dtype)), _bits(want_hk))
    assert np.array_equal(_bits(to_host_storage(hv, dtype)), _bits(want_hv))

    # the device blocks are reused meanwhile; the sequences come back into
    # blocks nobody holds (or the same ones), tables repointed
    used = set(int(b) for b in tables[tables >= 0].ravel())
    free = [b for b in range(w.num_blocks) if b not in used]
    rng = np.random.default_rng(2)
    dest = list(rng.permutation(free + blocks)[:len(blocks)])
    nan = float("nan")
    idx = torch.tensor(blocks, device="cuda", dtype=torch.long)
    g.k[idx] = nan
    g.v[idx] = nan
    in_pairs = np.stack([host_slot, dest], axis=1).astype(np.int32)
    pt = torch.from_numpy(in_pairs)
    pt = pt.pin_memory() if pairs_on_host else pt.cuda()
    k_mid = to_host_storage(g.k, dtype)
    v_mid = to_host_storage(g.v, dtype)
    pa.swap_blocks(g.k, g.v, hk, hv, pt)
    torch.cuda.synchronize()
    want_k, want_v = oracle.swap_blocks(k_mid, v_mid, want_hk, want_hv, in_pairs)
    assert np.array_equal(_bits(to_host_storage(g.k, dtype)), _bits(want_k))
    assert np.array_equal(_bits(to_host_storage(g.v, dtype)), _bits(want_v))

    # attention over the swapped-in blocks: same bits as before the swap
    remap = dict(zip(blocks, dest))
    t2 = tables.copy()
    for s in victims:
        nb = -(-int(w.context_lens[s]) // 16)
        t2[s, :nb] = [remap[int(b)] for b in tables[s, :nb]]
    after = pa.decode(g.q, g.k, g.v, torch.from_numpy(t2).cuda(), g.lens, w.scale, w.max_context_len)
    a = to_f64(out_before, dtype)
    b = to_f64(after, dtype)
    for s in victims:
        assert np.array_equal(a[s], b[s])


def test_device_to_device_and_skipped_ids():
    import torch

    import paged_kv_cache_117_amd as pa

    src_k = torch.randn(6, 2, 16, 64, device="cuda", dtype=torch.bfloat16)
    src_v = torch.randn_like(src_k)
    dst_k = torch.zeros(4, 2, 16, 64, device="cuda", dtype=torch.bfloat16)
    dst_v = torch.zeros_like(dst_k)
    pairs = torch.tensor([[5, 0], [2, 3], [6, 1], [0, 4], [-1, 2]], dtype=torch.int32, device="cuda")
    pa.swap_blocks(dst_k, dst_v, src_k, src_v, pairs)
    torch.cuda.synchronize()
    assert torch.equal(dst_k[0], src_k[5]) and torch.equal(dst_k[3], src_k[2])
    assert torch.equal(dst_v[0], src_v[5]) and torch.equal(dst_v[3], src_v[2])
    assert dst_k[1].abs().sum() == 0 and dst_k[2].abs().sum() == 0  # skipped pairs


def test_library_refuses_pageable_host_pool():
    """The C entry point checks the memory type before launching.  The only
    pair is out of range, so even a wrong verdict could not touch the pool."""
    import torch

    from paged_kv_cache_117_amd import _lib

    dev = torch.zeros(2, 2, 16, 64, device="cuda", dtype=torch.bfloat16)
    pageable = torch.zeros(2, 2, 16, 64, dtype=torch.bfloat16)
    pairs = torch.tensor([[-1, -1]], dtype=torch.int32, device="cuda")
    st = _lib.LIB.pa_swap_blocks(pageable.data_ptr(), pageable.data_ptr(), dev.data_ptr(), dev.data_ptr(),
                                 pairs.data_ptr(), 1, 2, 64, 16, 2, 2, _lib.PA_BF16, None)
    torch.cuda.synchronize()
    assert st == 2, _lib.LIB.pa_last_error()
    assert b"pinned" in _lib.LIB.pa_last_error() or b"accessible" in _lib.LIB.pa_last_error()
