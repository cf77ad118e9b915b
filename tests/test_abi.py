"""The C ABI: every declared function is exported and bound; host-side checks."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_117_amd as pa
from paged_kv_cache_117_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.SIGNATURES) == names


def test_abi_version():
    assert pa.abi_version() == 1


def _al(x):
    return (x + 255) // 256 * 256


def _even_split_bytes(B, Hq, Hkv, D):
    # 2 * 4096 piece slots of gmax rows (o [slot][gmax][D], m, l), then one
    # (slot, count) record per (sequence, KV head, query sub-group)
    g = Hq // Hkv
    gmax = 4 if g <= 4 else 8 if g <= 8 else 16
    nsub = -(-g // gmax)
    slots = 2 * 4096
    return _al(slots * gmax * D * 4) + 2 * _al(slots * gmax * 4) + _al(B * Hkv * nsub * 8)


def test_workspace_bytes():
    # batches of up to 4096 sequences: the even split's pieces (any length)
    assert pa.decode_workspace_bytes(4, 2, 2, 64, 37, 0) == _even_split_bytes(4, 2, 2, 64)
    assert pa.decode_workspace_bytes(64, 32, 8, 128, 512, 512) == _even_split_bytes(64, 32, 8, 128)
    assert pa.decode_workspace_bytes(7, 40, 40, 128, 100, 0) == _even_split_bytes(7, 40, 40, 128)
    assert pa.decode_workspace_bytes(2, 64, 2, 64, 100, 0) == _even_split_bytes(2, 64, 2, 64)
    # or the partitions' partials when larger: 8 partitions of 512 for 4096
    # tokens, o [B][Hq][P][D] + m + l, each 256-aligned
    rows = 4096 * 32 * 8
    assert pa.decode_workspace_bytes(4096, 32, 8, 128, 4096, 0) == rows * 128 * 4 + 2 * rows * 4
    # more than 4096 sequences: partitions only (none when one partition fits)
    assert pa.decode_workspace_bytes(5000, 32, 8, 128, 512, 0) == 0
    rows = 5000 * 32 * 2
    assert pa.decode_workspace_bytes(5000, 32, 8, 128, 1024, 512) == rows * 128 * 4 + 2 * _al(rows * 4)
    assert pa.decode_workspace_bytes(0, 32, 8, 128, 4096, 0) == 0
    assert pa.decode_workspace_bytes(4, 32, 5, 128, 4096, 0) == 0


L = _lib.LIB
NULL = None


def call_decode(**kw):
    a = dict(out=16, q=16, k=16, v=16, bt=16, cl=16, B=1, Hq=2, Hkv=2, D=64, bs=16, nb=4, maxb=2,
             maxctx=20, scale=0.125, dt=0, ps=0, ws=NULL, wsb=0, stream=NULL)
    a.update(kw)
    return L.pa_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["B"], a["Hq"], a["Hkv"], a["D"],
                       a["bs"], a["nb"], a["maxb"], a["maxctx"], a["scale"], a["dt"], a["ps"], a["ws"], a["wsb"],
                       a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bs=8), 3), (dict(bs=48), 3), (dict(bs=256), 3), (dict(D=96), 3), (dict(dt=7), 3),
    (dict(Hq=3, Hkv=2), 2), (dict(maxctx=33), 2), (dict(ps=24), 2), (dict(B=-1), 2),
    (dict(scale=float("inf")), 2), (dict(q=NULL), 1), (dict(out=8), 2),
    (dict(maxctx=600, maxb=64), 4), (dict(dt=2), 4), (dict(dt=1, wsb=64, ws=256), 4),
])
def test_decode_host_validation(kw, status):
    """Rejected before any device work (these calls never reach the GPU)."""
    assert call_decode(**kw) == status
    assert L.pa_last_error().decode()


def test_decode_zero_sequences_is_a_no_op():
    assert call_decode(B=0, out=NULL, q=NULL) == 0


def test_write_and_copy_host_validation():
    assert L.pa_write_kv(16, 16, 16, 16, 16, 1, 2, 64, 24, 4, 0, NULL) == 3  # block size not a power of two
    assert L.pa_write_kv(16, 16, 16, 16, NULL, 1, 2, 64, 16, 4, 0, NULL) == 1
    assert L.pa_write_kv(16, 16, 8, 16, 16, 1, 2, 64, 16, 4, 0, NULL) == 2
    assert L.pa_write_kv(NULL, NULL, NULL, NULL, NULL, 0, 2, 64, 16, 4, 0, NULL) == 0
    assert L.pa_copy_blocks(16, 16, 16, 1, 2, 100, 16, 4, 0, NULL) == 3
    assert L.pa_copy_blocks(16, 16, NULL, 1, 2, 64, 16, 4, 0, NULL) == 1
    assert L.pa_copy_blocks(NULL, NULL, NULL, 0, 2, 64, 16, 4, 0, NULL) == 0


def test_binding_refuses_host_tensors():
    import torch

    q = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError):
        pa.decode(q, torch.zeros(4, 2, 16, 64), torch.zeros(4, 2, 16, 64),
                  torch.zeros(1, 2, dtype=torch.int32), torch.ones(1, dtype=torch.int32), 0.125, 1)


def test_one_hip_runtime_in_the_process():
    """libpa binds to torch's HIP runtime; a second copy would not see the device."""
    maps = [line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line]
    assert len(set(maps)) == 1, sorted(set(maps))


def call_prefill(**kw):
    a = dict(out=16, q=16, k=16, v=16, bt=16, cl=16, qs=16, B=1, N=4, Hq=2, Hkv=2, D=64, bs=16, nb=4, maxb=2,
             maxq=4, maxctx=20, ps=0, scale=0.125, dt=2, ws=NULL, wsb=0, stream=NULL)
    a.update(kw)
    return L.pa_prefill(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["qs"], a["B"], a["N"], a["Hq"],
                        a["Hkv"], a["D"], a["bs"], a["nb"], a["maxb"], a["maxq"], a["maxctx"], a["ps"], a["scale"],
                        a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bs=4), 3), (dict(bs=256), 3), (dict(D=96), 3), (dict(dt=7), 3), (dict(dt=0, bs=8), 3),
    (dict(Hq=3, Hkv=2), 2), (dict(maxq=5), 2), (dict(N=-1), 2), (dict(B=-1), 2), (dict(nb=0), 2),
    (dict(scale=float("nan")), 2), (dict(qs=NULL), 1), (dict(q=NULL), 1), (dict(out=8), 2),
    (dict(maxctx=33), 2), (dict(ps=-1), 2), (dict(maxctx=200, maxb=16, ps=64), 4),
    (dict(maxctx=200, maxb=16, ps=64, wsb=64, ws=256), 4), (dict(maxctx=200, maxb=16, ps=64, wsb=1 << 20, ws=8), 4),
])
def test_prefill_host_validation(kw, status):
    """Rejected before any device work (these calls never reach the GPU: every
    case must fail a host check, the pointers are not real)."""
    assert call_prefill(**kw) == status
    assert L.pa_last_error().decode()


def test_prefill_without_rows_is_a_no_op():
    assert call_prefill(N=0, maxq=0, out=NULL, q=NULL, qs=NULL) == 0
    assert call_prefill(B=0, out=NULL, q=NULL) == 0


def test_swap_host_validation():
    """Checks that come before any pointer query or launch."""
    sw = L.pa_swap_blocks
    assert sw(16, 16, 16, 16, 16, 1, 2, 64, 16, 4, 4, 7, NULL) == 3   # dtype
    assert sw(16, 16, 16, 16, 16, 1, 2, 64, 256, 4, 4, 2, NULL) == 3  # block size
    assert sw(16, 16, 16, 16, 16, 1, 2, 96, 16, 4, 4, 2, NULL) == 3   # head dim
    assert sw(16, 16, 16, 16, 16, -1, 2, 64, 16, 4, 4, 2, NULL) == 2  # negative count
    assert sw(16, 16, NULL, 16, 16, 1, 2, 64, 16, 4, 4, 2, NULL) == 1
    assert sw(16, 16, 8, 16, 16, 1, 2, 64, 16, 4, 4, 2, NULL) == 2    # misaligned
    assert sw(NULL, NULL, NULL, NULL, NULL, 0, 2, 64, 16, 4, 4, 2, NULL) == 0


def test_swap_binding_refuses_pageable_host_pools():
    import torch

    pool = torch.zeros(4, 2, 16, 64)
    with pytest.raises(ValueError):
        pa.swap_blocks(pool, pool.clone(), pool.clone(), pool.clone(), torch.zeros(1, 2, dtype=torch.int32))


def test_prefill_workspace_bytes():
    # unsplit launches need none: many workgroups, or short contexts
    assert pa.prefill_workspace_bytes(8, 4096, 32, 8, 128, 512, 3704, 0) == 0
    assert pa.prefill_workspace_bytes(4, 256, 32, 8, 128, 64, 500, 0) == 0
    # a short chunk over a long context: 4 seqs x 8 heads x 2 tiles = 64 groups -> 8 partitions
    rows = 256 * 32 * 8
    assert pa.prefill_workspace_bytes(4, 256, 32, 8, 128, 64, 32768, 0) == _al(rows * 128 * 4) + 2 * _al(rows * 4)
    # a given partition size always splits: ceil(32768 / 1024) = 32 partitions
    rows = 256 * 32 * 32
    assert pa.prefill_workspace_bytes(4, 256, 32, 8, 128, 64, 32768, 1000) == _al(rows * 128 * 4) + 2 * _al(rows * 4)
    assert pa.prefill_workspace_bytes(0, 256, 32, 8, 128, 64, 32768, 0) == 0


def test_time_next_main_kernel_argument_rules():
    # one event without the other is refused; none cancels (nothing is launched here)
    assert L.pa_time_next_main_kernel(None, 12345) == 1  # PA_ERR_NULL
    assert b"both" in L.pa_last_error()
    assert L.pa_time_next_main_kernel(None, None) == 0
    pa.time_next_main_kernel(None, None)
    with pytest.raises(TypeError):
        pa.time_next_main_kernel(1, 2)


def test_decode_noalloc_host_validation():
    """pa_decode_noalloc checks arguments like pa_decode, and refuses sizes
    whose partials exceed its scratch before touching the device."""
    import ctypes

    from paged_kv_cache_117_amd._lib import LIB

    p = 4096  # never dereferenced: every call below fails on the host
    st = LIB.pa_decode_noalloc(p, p, p, p, p, p, 4096, 64, 8, 128, 16, 1, 512, 8192, ctypes.c_float(0.1), 0, 512, None)
    assert st == 4 and "scratch" in LIB.pa_last_error().decode()
    st = LIB.pa_decode_noalloc(p, p, p, p, p, p, 4, 8, 2, 128, 4, 1, 8, 64, ctypes.c_float(0.1), 2, 0, None)
    assert st == 3  # block size 4
    st = LIB.pa_decode_noalloc(p, p, p, p, p, p, 4, 8, 2, 128, 8, 1, 8, 64, ctypes.c_float(0.1), 0, 0, None)
    assert st == 3  # block size 8 with fp32 KV
    st = LIB.pa_decode_noalloc(None, p, p, p, p, p, 4, 8, 2, 128, 16, 1, 8, 64, ctypes.c_float(0.1), 2, 0, None)
    assert st == 1
    assert LIB.pa_decode_noalloc(p, p, p, p, p, p, 0, 8, 2, 128, 16, 1, 8, 64, ctypes.c_float(0.1), 2, 0, None) == 0


def test_probe_read_host_validation():
    """pa_probe_read refuses bad modes, sizes and pointers on the host (the
    fake pointer below is never dereferenced: every call fails before a
    launch)."""
    p = 4096
    assert L.pa_probe_read(p, 8192, p, 2, 2, 1, p, None) == 3  # mode
    assert L.pa_probe_read(p, 4095, None, 0, 0, 1, p, None) == 2  # not whole 4 KiB chunks
    assert L.pa_probe_read(p, 0, None, 0, 0, 1, p, None) == 2
    assert L.pa_probe_read(p, 8192, None, 0, 0, 0, p, None) == 2  # workgroups
    assert L.pa_probe_read(p + 8, 8192, None, 0, 0, 1, p, None) == 2  # alignment
    assert L.pa_probe_read(None, 8192, None, 0, 0, 1, p, None) == 1
    assert L.pa_probe_read(p, 8192, None, 4, 1, 1, p, None) == 1  # gather without an order
    assert L.pa_probe_read(p, 8192, p, -1, 1, 1, p, None) == 2
