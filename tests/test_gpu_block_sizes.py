"""Block sizes other than 16 (PagedAttention and vLLM: Paging the KV Cache
Like an OS, "Why 16 tokens"; PagedAttention: Virtual Memory for the KV Cache,
"Block size: why 16").  The decode kernels walk 16-slot tiles, so pa_decode
takes blocks of 16, 32, 64 or 128 slots; pa_prefill also takes 8; the data
movement (write, copy, swap) any power of two up to 128.  Every case is the
whole step against the oracle, whose gather follows the pool's block size."""

import numpy as np
import pytest

import oracle
from harness import TOL, GpuPrefillStep, GpuStep, oracle_prefill_pools, oracle_step, to_device, to_f64, \
    to_host_storage
from workloads import make_custom, make_prefill_custom

pytestmark = pytest.mark.gpu


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype.itemsize == 2 else a.view(np.uint32)


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype,hq,hkv,d,psize", [("bf16", 32, 8, 128, 0), ("fp16", 16, 2, 64, 256),
                                                   ("fp16", 8, 8, 128, 2048), ("fp32", 4, 2, 64, 0)])
def test_decode_and_write(bs, dtype, hq, hkv, d, psize):
    lens = [1, 15, 16, 17, 33, 127, 128, 129, 300, 1000, 2049]
    w = make_custom(f"bs{bs}", dtype, lens, hq, hkv, d, seed=500 + bs, block_size=bs)
    print(f"case decode bs={bs} {dtype} psize={psize}", flush=True)
    g = GpuStep(w)
    out = to_f64(g.run(partition_size=psize), dtype)
    st, k, v, want = oracle_step(w)
    assert np.array_equal(_bits(to_host_storage(g.k, dtype)), _bits(k))
    assert np.array_equal(_bits(to_host_storage(g.v, dtype)), _bits(v))
    assert np.isfinite(out).all()
    assert np.abs(out - want).max() <= TOL[dtype]


def test_decode_refuses_blocks_below_16():
    import paged_kv_cache_117_amd as pa

    w = make_custom("bs8", "bf16", [20, 40], 8, 2, 64, seed=7, block_size=8)
    g = GpuStep(w)
    with pytest.raises(pa.PaError):
        g.run()


@pytest.mark.parametrize("bs", [8, 32, 128])
def test_prefill(bs):
    w = make_prefill_custom(f"pbs{bs}", "bf16", [0, 37, 130, 5], [45, 70, 1, 200], 16, 4, 128, seed=600 + bs,
                            block_size=bs)
    print(f"case prefill bs={bs}", flush=True)
    g = GpuPrefillStep(w)
    out = to_f64(g.run(), "bf16")
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    assert np.isfinite(out).all()
    assert np.abs(out - want).max() <= TOL["bf16"]


@pytest.mark.parametrize("bs", [1, 4, 8, 32, 128])
def test_copy_and_swap_blocks(bs):
    import torch

    import paged_kv_cache_117_amd as pa

    rng = np.random.default_rng(bs)
    nb, hkv, d = 40, 2, 64
    k = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
    v = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:10], perm[10:20]], axis=1).astype(np.int32)
    kd, vd = to_device(k, "fp16"), to_device(v, "fp16")
    pa.copy_blocks(kd, vd, torch.from_numpy(pairs).cuda())
    wk, wv = oracle.copy_blocks(k, v, pairs)
    assert np.array_equal(_bits(to_host_storage(kd, "fp16")), _bits(wk))
    assert np.array_equal(_bits(to_host_storage(vd, "fp16")), _bits(wv))
    hk = torch.zeros((12, hkv, bs, d), dtype=torch.float16, pin_memory=True)
    hv = torch.zeros_like(hk, pin_memory=True)
    sp = np.stack([perm[20:32], np.arange(12)], axis=1).astype(np.int32)
    pa.swap_blocks(hk, hv, kd, vd, torch.from_numpy(sp).cuda())
    torch.cuda.synchronize()
    ok, ov = oracle.swap_blocks(np.zeros((12, hkv, bs, d), np.float16), np.zeros((12, hkv, bs, d), np.float16),
                                wk, wv, sp)
    assert np.array_equal(_bits(hk.numpy()), _bits(ok)) and np.array_equal(_bits(hv.numpy()), _bits(ov))
