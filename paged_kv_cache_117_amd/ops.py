"""Python binding of the device entry points: argument marshalling only.

Every call checks what the C ABI cannot see (tensor devices, dtypes, shapes,
contiguity), so that the kernels only ever receive device buffers of the sizes
the sizes arguments describe, then calls straight into libpa.so.  All work
runs in the library's HIP kernels on the current (or given) stream.
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import LIB, PA_BF16, PA_ERR_NO_BLOCKS, PA_FP16, PA_FP32, STATUS_NAMES

BLOCK_SIZE = 16
_DTYPES = {torch.float32: PA_FP32, torch.float16: PA_FP16, torch.bfloat16: PA_BF16}


class PaError(RuntimeError):
    def __init__(self, msg, status):
        super().__init__(msg)
        self.status = status


class NoFreeBlocks(PaError):
    pass


def check_status(st: int, what: str) -> None:
    if st != 0:
        msg = LIB.pa_last_error().decode(errors="replace")
        cls = NoFreeBlocks if st == PA_ERR_NO_BLOCKS else PaError
        raise cls(f"{what}: {STATUS_NAMES.get(st, st)}: {msg}", st)


def _device_tensor(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, current device is {torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t


def _stream_handle(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _launch_stream(stream):
    """The torch stream the library launches on (current, given, or a raw
    hipStream_t handle wrapped without taking ownership).  Temporaries the
    binding allocates for a call are allocated on it, so torch's caching
    allocator does not hand their memory to other work while the call's
    kernels still use it."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _alloc_on(ts, fn):
    """fn() with `ts` current, so its allocations belong to `ts`."""
    if ts == torch.cuda.current_stream():
        return fn()
    with torch.cuda.stream(ts):
        return fn()


def _dtype_code(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_context_len: int, partition_size: int = 0) -> int:
    return int(LIB.pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                             partition_size))


def decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, max_context_len: int,
           out=None, partition_size: int = 0, workspace=None, stream=None):
    """Paged decode attention (pa_decode).  Returns ``out`` [B][Hq][D]."""
    _device_tensor(q, "q", ndim=3)
    B, Hq, D = q.shape
    _device_tensor(k_pool, "k_pool", q.dtype, 4)
    _device_tensor(v_pool, "v_pool", q.dtype, 4)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool shapes differ")
    nb, Hkv, bs, Dk = k_pool.shape
    if Dk != D:
        raise ValueError(f"head_dim mismatch: q {D}, pools {Dk}")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens rows must equal num_seqs")
    ts = _launch_stream(stream)
    if out is None:
        out = _alloc_on(ts, lambda: torch.empty_like(q))
    _device_tensor(out, "out", q.dtype, 3)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, partition_size)
    if workspace is None and need:
        workspace = _alloc_on(ts, lambda: torch.empty(need, dtype=torch.uint8, device=q.device))
    if workspace is not None:
        _device_tensor(workspace, "workspace")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = LIB.pa_decode(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                       block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, D, bs, nb,
                       block_tables.shape[1], int(max_context_len), float(scale), _dtype_code(q),
                       int(partition_size), ws_ptr, ws_bytes, ts.cuda_stream)
    check_status(st, "pa_decode")
    return out


def write_kv_decode(q, k_pool, v_pool, k_new, v_new, block_tables, context_lens, scale: float, max_context_len: int,
                    out=None, partition_size: int = 0, workspace=None, stream=None):
    """One decode step in one call (pa_write_kv_decode): each sequence's new
    K/V rows are stored at its last position through its block table and
    attended to.  Returns ``out`` [B][Hq][D]."""
    _device_tensor(q, "q", ndim=3)
    B, Hq, D = q.shape
    _device_tensor(k_pool, "k_pool", q.dtype, 4)
    _device_tensor(v_pool, "v_pool", q.dtype, 4)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool shapes differ")
    nb, Hkv, bs, Dk = k_pool.shape
    if Dk != D:
        raise ValueError(f"head_dim mismatch: q {D}, pools {Dk}")
    _device_tensor(k_new, "k_new", q.dtype, 3)
    _device_tensor(v_new, "v_new", q.dtype, 3)
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError(f"k_new/v_new must be [{B}][{Hkv}][{D}]")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens rows must equal num_seqs")
    ts = _launch_stream(stream)
    if out is None:
        out = _alloc_on(ts, lambda: torch.empty_like(q))
    _device_tensor(out, "out", q.dtype, 3)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, partition_size)
    if workspace is None and need:
        workspace = _alloc_on(ts, lambda: torch.empty(need, dtype=torch.uint8, device=q.device))
    if workspace is not None:
        _device_tensor(workspace, "workspace")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = LIB.pa_write_kv_decode(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(),
                                v_new.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, D, bs,
                                nb, block_tables.shape[1], int(max_context_len), float(scale), _dtype_code(q),
                                int(partition_size), ws_ptr, ws_bytes, ts.cuda_stream)
    check_status(st, "pa_write_kv_decode")
    return out


def prefill_workspace_bytes(num_seqs: int, num_tokens: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            max_query_len: int, max_context_len: int, partition_size: int = 0) -> int:
    return int(LIB.pa_prefill_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                              max_query_len, max_context_len, partition_size))


def prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale: float, max_query_len: int,
            max_context_len: int, out=None, partition_size: int = 0, workspace=None, stream=None):
    """Paged attention for a chunk of new tokens per sequence (pa_prefill).

    ``q`` is [N][Hq][D] with sequence s owning rows query_start[s] ..
    query_start[s+1]-1; returns ``out`` of q's shape.
    """
    _device_tensor(q, "q", ndim=3)
    N, Hq, D = q.shape
    _device_tensor(k_pool, "k_pool", q.dtype, 4)
    _device_tensor(v_pool, "v_pool", q.dtype, 4)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool shapes differ")
    nb, Hkv, bs, Dk = k_pool.shape
    if Dk != D:
        raise ValueError(f"head_dim mismatch: q {D}, pools {Dk}")
    _device_tensor(block_tables, "block_tables", torch.int32, 2)
    _device_tensor(context_lens, "context_lens", torch.int32, 1)
    _device_tensor(query_start, "query_start", torch.int32, 1)
    B = context_lens.shape[0]
    if block_tables.shape[0] != B or query_start.shape[0] != B + 1:
        raise ValueError("block_tables rows must equal num_seqs and query_start must have num_seqs + 1 entries")
    ts = _launch_stream(stream)
    if out is None:
        out = _alloc_on(ts, lambda: torch.empty_like(q))
    _device_tensor(out, "out", q.dtype, 3)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = prefill_workspace_bytes(B, N, Hq, Hkv, D, max_query_len, max_context_len, partition_size)
    if workspace is None and need:
        workspace = _alloc_on(ts, lambda: torch.empty(need, dtype=torch.uint8, device=q.device))
    if workspace is not None:
        _device_tensor(workspace, "workspace")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = LIB.pa_prefill(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                        block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(), B, N, Hq,
                        Hkv, D, bs, nb, block_tables.shape[1], int(max_query_len), int(max_context_len),
                        int(partition_size), float(scale), _dtype_code(q), ws_ptr, ws_bytes, ts.cuda_stream)
    check_status(st, "pa_prefill")
    return out


def write_kv(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None):
    """Store new tokens' K/V rows at their slots (pa_write_kv)."""
    _device_tensor(k_pool, "k_pool", ndim=4)
    _device_tensor(v_pool, "v_pool", k_pool.dtype, 4)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool shapes differ")
    nb, Hkv, bs, D = k_pool.shape
    _device_tensor(k_new, "k_new", k_pool.dtype, 3)
    _device_tensor(v_new, "v_new", k_pool.dtype, 3)
    _device_tensor(slot_mapping, "slot_mapping", torch.int64, 1)
    T = slot_mapping.shape[0]
    if tuple(k_new.shape) != (T, Hkv, D) or tuple(v_new.shape) != (T, Hkv, D):
        raise ValueError(f"k_new/v_new must be [{T}][{Hkv}][{D}]")
    st = LIB.pa_write_kv(k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                         slot_mapping.data_ptr(), T, Hkv, D, bs, nb, _dtype_code(k_pool),
                         _stream_handle(stream))
    check_status(st, "pa_write_kv")


def copy_blocks(k_pool, v_pool, block_pairs, stream=None):
    """Whole-block copies (src -> dst) for copy-on-write (pa_copy_blocks)."""
    _device_tensor(k_pool, "k_pool", ndim=4)
    _device_tensor(v_pool, "v_pool", k_pool.dtype, 4)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool shapes differ")
    nb, Hkv, bs, D = k_pool.shape
    _device_tensor(block_pairs, "block_pairs", torch.int32, 2)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n][2]")
    st = LIB.pa_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), block_pairs.data_ptr(),
                            block_pairs.shape[0], Hkv, D, bs, nb, _dtype_code(k_pool),
                            _stream_handle(stream))
    check_status(st, "pa_copy_blocks")


def _pool_tensor(t, name, dtype=None):
    """A pool on the GPU or in pinned host memory (the library checks which)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.is_cuda:
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name} is on {t.device}, current device is {torch.cuda.current_device()}")
    elif not t.is_pinned():
        raise ValueError(f"{name} lives in pageable host memory; allocate it with pin_memory=True")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must have 4 dims, got shape {tuple(t.shape)}")
    return t


def swap_blocks(dst_k, dst_v, src_k, src_v, block_pairs, stream=None):
    """Whole-block copies src[pair[0]] -> dst[pair[1]] between a device pool
    and a pinned host pool (pa_swap_blocks): swap-out or swap-in."""
    _pool_tensor(src_k, "src_k")
    for n, t in (("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v)):
        _pool_tensor(t, n, src_k.dtype)
    if src_k.shape != src_v.shape or dst_k.shape != dst_v.shape or src_k.shape[1:] != dst_k.shape[1:]:
        raise ValueError("pools must share the block shape (K and V alike)")
    if not isinstance(block_pairs, torch.Tensor) or block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 \
            or block_pairs.shape[1] != 2 or not block_pairs.is_contiguous():
        raise ValueError("block_pairs must be a contiguous int32 [n][2] tensor")
    if not block_pairs.is_cuda and not block_pairs.is_pinned():
        raise ValueError("block_pairs must be on the GPU or in pinned host memory")
    ns, Hkv, bs, D = src_k.shape
    st = LIB.pa_swap_blocks(dst_k.data_ptr(), dst_v.data_ptr(), src_k.data_ptr(), src_v.data_ptr(),
                            block_pairs.data_ptr(), block_pairs.shape[0], Hkv, D, bs, ns, dst_k.shape[0],
                            _dtype_code(src_k), _stream_handle(stream))
    check_status(st, "pa_swap_blocks")


def abi_version() -> int:
    return int(LIB.pa_abi_version())


def time_next_main_kernel(start, stop) -> None:
    """pa_time_next_main_kernel: the next decode / prefill call records the
    two torch.cuda.Event objects (timing enabled) right around its main
    kernel; ``start.elapsed_time(stop)`` is then that kernel's duration.
    None, None cancels a pending request."""
    if start is None and stop is None:
        check_status(LIB.pa_time_next_main_kernel(None, None), "pa_time_next_main_kernel")
        return
    handles = []
    for ev in (start, stop):
        if not isinstance(ev, torch.cuda.Event):
            raise TypeError("start and stop must be torch.cuda.Event objects")
        if not ev.cuda_event:
            ev.record()  # torch creates the underlying event on its first record
        handles.append(ev.cuda_event)
    check_status(LIB.pa_time_next_main_kernel(handles[0], handles[1]), "pa_time_next_main_kernel")


def probe_read(buf, sink, workgroups: int, chunk_order=None, stream=None) -> None:
    """pa_probe_read: read ``buf`` (a contiguous device tensor of a multiple of
    4096 bytes) sequentially (``chunk_order`` None) or as whole 4 KiB chunks
    in the order ``chunk_order`` (device int32) gives; ``sink`` is a device
    int32 tensor of at least ``workgroups * 256`` elements."""
    _device_tensor(buf, "buf")
    _device_tensor(sink, "sink", torch.int32)
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < workgroups * 256:
        raise ValueError(f"sink holds {sink.numel()} words, the launch writes {workgroups * 256}")
    if chunk_order is None:
        mode, order, n = 0, None, 0
    else:
        _device_tensor(chunk_order, "chunk_order", torch.int32, 1)
        mode, order, n = 1, chunk_order.data_ptr(), chunk_order.numel()
    check_status(LIB.pa_probe_read(buf.data_ptr(), nbytes, order, n, mode, int(workgroups), sink.data_ptr(),
                                   _stream_handle(stream)), "pa_probe_read")


def _as_ptr(arr, ctype):
    return arr.ctypes.data_as(ctypes.POINTER(ctype))
