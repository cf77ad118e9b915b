"""Block sizes other than 16 (PagedAttention and vLLM: Paging the KV Cache
Like an OS, "Why 16 tokens"; PagedAttention: Virtual Memory for the KV Cache,
"Block size: why 16").  The decode kernels walk 16-slot tiles, so pa_decode
runs blocks of 16, 32, 64 or 128 slots on them and blocks of 8 (16-bit KV)
through the prefill kernel, which walks token rows; pa_prefill takes 8 to
128; the data movement (write, copy, swap) any power of two up to 128.  Every
case is the whole step against the oracle, whose gather follows the pool's
block size."""

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


SHAPES = [("bf16", 32, 8, 128, 0), ("fp16", 16, 2, 64, 256), ("fp16", 8, 8, 128, 2048), ("fp32", 4, 2, 64, 0)]


@pytest.mark.parametrize("bs,dtype,hq,hkv,d,psize",
                         [(bs,) + sh for bs in (8, 16, 32, 64, 128) for sh in SHAPES if not (bs == 8 and sh[0] == "fp32")])
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


def test_decode_refuses_fp32_blocks_of_8_and_blocks_below_8():
    import paged_kv_cache_117_amd as pa

    g = GpuStep(make_custom("bs8f32", "fp32", [20, 40], 8, 2, 64, seed=7, block_size=8))
    with pytest.raises(pa.PaError):
        g.run()
    g = GpuStep(make_custom("bs4", "bf16", [20, 40], 8, 2, 64, seed=7, block_size=4))
    with pytest.raises(pa.PaError):
        g.run()


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("fp16", 64, 8, 128), ("fp16", 40, 40, 64)])
def test_decode_blocks_of_8_edges_fused_and_noalloc(dtype, hq, hkv, d):
    """Blocks of 8 slots: L = 0 gives a zero row, L beyond max_context_len
    and a bad block id NaN rows (as with larger blocks); pa_write_kv_decode
    equals pa_write_kv + pa_decode bit for bit; pa_decode_noalloc equals
    pa_decode bit for bit; and the split launch (a short batch, long
    contexts) and the unsplit one both match the oracle on every row."""
    import torch

    import paged_kv_cache_117_amd as pa

    lens = [1, 7, 8, 9, 40, 600, 2500, 41]
    w = make_custom(f"bs8{dtype}{hq}", dtype, lens, hq, hkv, d, seed=31 + hq, block_size=8)
    print(f"case decode bs=8 {dtype} hq={hq} hkv={hkv} d={d}", flush=True)
    g = GpuStep(w)
    kf, vf = g.k.clone(), g.v.clone()
    for psize in (0, 512):
        out = to_f64(g.run(partition_size=psize), dtype)
        st, k, v, want = oracle_step(w)
        assert np.isfinite(out).all()
        assert np.abs(out - want).max() <= TOL[dtype]
    ref = g.out.clone()
    # the fused step from the same pre-step pools
    if len(g.st.pairs):
        pa.copy_blocks(kf, vf, g.pairs)
    of = pa.write_kv_decode(g.q, kf, vf, g.k_new, g.v_new, g.tables, g.lens, w.scale, w.max_context_len,
                            partition_size=512)
    torch.cuda.synchronize()
    assert torch.equal(of.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(kf.view(torch.int16), g.k.view(torch.int16))
    assert torch.equal(vf.view(torch.int16), g.v.view(torch.int16))
    # the allocation-free entry point, twice
    import ctypes

    from paged_kv_cache_117_amd._lib import LIB

    for _ in range(2):
        on = torch.full_like(ref, float("nan"))
        st = LIB.pa_decode_noalloc(on.data_ptr(), g.q.data_ptr(), g.k.data_ptr(), g.v.data_ptr(), g.tables.data_ptr(),
                                   g.lens.data_ptr(), w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, 8,
                                   w.num_blocks, g.tables.shape[1], w.max_context_len, ctypes.c_float(w.scale),
                                   {"fp16": 1, "bf16": 2}[dtype], 512, torch.cuda.current_stream().cuda_stream)
        assert st == 0, LIB.pa_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(on.view(torch.int16), ref.view(torch.int16))
    # edges: zero length, a length past max_context_len, a bad block id
    lens2 = g.lens.clone()
    lens2[0] = 0
    lens2[1] = w.max_context_len + 1
    tables2 = g.tables.clone()
    tables2[2, 0] = w.num_blocks + 3
    o = pa.decode(g.q, g.k, g.v, tables2, lens2, w.scale, w.max_context_len).float().cpu().numpy()
    assert np.all(o[0] == 0)
    assert np.all(np.isnan(o[1]))
    assert np.all(np.isnan(o[2]))
    keep = list(range(3, len(lens)))
    assert np.abs(o[keep] - want[keep]).max() <= TOL[dtype]


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
