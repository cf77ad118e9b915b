"""GPU: pa_decode_noalloc (partials in the library's own device scratch)
against pa_decode with a caller workspace, through the C ABI.

Both entry points launch the same kernels with the same split, so their
outputs must agree bit for bit; each is also held to the fp64 oracle's
tolerance.  Two calls in a row, the second on a smaller input, show that the
scratch's leftovers from one call do not leak into the next.
"""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_117_amd as pa
from harness import TOL, GpuStep, oracle_step, to_f64
from paged_kv_cache_117_amd._lib import LIB, PA_BF16, PA_FP16, PA_FP32, STATUS_NAMES
from workloads import make_custom

pytestmark = pytest.mark.gpu

CODES = {"fp32": PA_FP32, "fp16": PA_FP16, "bf16": PA_BF16}
PA_ERR_WORKSPACE = 4


def noalloc(g, partition_size, out):
    w = g.w
    st = LIB.pa_decode_noalloc(out.data_ptr(), g.q.data_ptr(), g.k.data_ptr(), g.v.data_ptr(), g.tables.data_ptr(),
                               g.lens.data_ptr(), w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                               w.block_size, w.num_blocks, g.tables.shape[1], w.max_context_len,
                               ctypes.c_float(w.scale), CODES[w.dtype], partition_size,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"pa_decode_noalloc: {STATUS_NAMES.get(st, st)}: {LIB.pa_last_error().decode()}"
    return out


def with_workspace(g, partition_size):
    w = g.w
    need = pa.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                                     partition_size)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(g.q)
    st = LIB.pa_decode(out.data_ptr(), g.q.data_ptr(), g.k.data_ptr(), g.v.data_ptr(), g.tables.data_ptr(),
                       g.lens.data_ptr(), w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                       w.num_blocks, g.tables.shape[1], w.max_context_len, ctypes.c_float(w.scale), CODES[w.dtype],
                       partition_size, ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"pa_decode: {STATUS_NAMES.get(st, st)}: {LIB.pa_last_error().decode()}"
    return out


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


CASES = [
    # (dtype, Hq, Hkv, D, lengths of the first call, lengths of the second (smaller) call, partition size)
    ("bf16", 32, 8, 128, list(range(128, 4097, 63)), [17, 300, 1, 2049, 64], 0),
    ("fp16", 64, 8, 128, [4096, 8192, 5000, 6100, 7777, 4097], [513, 1024, 40], 512),
    ("fp16", 40, 40, 128, [64, 2048, 700, 1500, 999], [5, 70], 0),
    ("fp32", 2, 2, 64, [1, 5, 16, 37, 1100, 2049], [3, 600], 0),
]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,lens1,lens2,psize", CASES)
def test_noalloc_matches_workspace_entry_point_twice(dtype, Hq, Hkv, D, lens1, lens2, psize):
    for call, lens in enumerate((lens1, lens2)):
        w = make_custom(f"noalloc{call}", dtype, lens, Hq, Hkv, D, seed=50 + call + D + Hq)
        print(f"[noalloc] call {call}: {dtype} B={w.num_seqs} Hq={Hq} Hkv={Hkv} D={D} psize={psize}", flush=True)
        g = GpuStep(w)
        g.run(partition_size=psize)  # the step's copies and writes (and a first decode)
        torch.cuda.synchronize()
        ref = with_workspace(g, psize)
        got = noalloc(g, psize, torch.full_like(g.q, float("nan")))
        torch.cuda.synchronize()
        assert torch.equal(bits(ref), bits(got))
        _, _, _, want = oracle_step(w)
        err = float(np.max(np.abs(to_f64(got, dtype) - want)))
        assert np.all(np.isfinite(to_f64(got, dtype))) and err <= TOL[dtype], err


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """fp32 KV with many sequences and partitions needs more partial space
    than the scratch holds: refused before anything is launched."""
    B, Hq, D, L = 4096, 64, 128, 8192
    dummy = torch.empty(16, dtype=torch.float32, device="cuda")
    p = dummy.data_ptr()
    st = LIB.pa_decode_noalloc(p, p, p, p, p, p, B, Hq, 8, D, 16, 1, L // 16, L, ctypes.c_float(0.1), PA_FP32, 512,
                               None)
    assert st == PA_ERR_WORKSPACE
    assert "scratch" in LIB.pa_last_error().decode()
