"""ctypes loader for libpa.so.  Raises ImportError when the library is missing."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIB_PATH names another build of the same library (the host-sanitizer run
# links one under _build/san); the in-tree libpa.so otherwise.
LIB_PATH = os.environ.get("PA_LIB_PATH") or os.path.join(HERE, "libpa.so")

PA_FP32, PA_FP16, PA_BF16 = 0, 1, 2
PA_OK = 0
PA_ERR_NO_BLOCKS = 6
STATUS_NAMES = {
    0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED", 4: "PA_ERR_WORKSPACE",
    5: "PA_ERR_LAUNCH", 6: "PA_ERR_NO_BLOCKS", 7: "PA_ERR_NOT_FOUND", 8: "PA_ERR_EXISTS",
}

_c = ctypes
_vp, _i32, _i64, _f32, _sz = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_float, _c.c_size_t
_pi32 = _c.POINTER(_c.c_int32)
_pi64 = _c.POINTER(_c.c_int64)

# name -> (restype, argtypes); one entry per function declared in include/pa.h
SIGNATURES = {
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                         _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_write_kv_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _i32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _f32, _i32, _i32, _vp]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                          _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_prefill_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_write_kv": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_swap_blocks": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_last_error": (_c.c_char_p, []),
    "pa_abi_version": (_i32, []),
    "pa_time_next_main_kernel": (_i32, [_vp, _vp]),
    "pa_probe_read": (_i32, [_vp, _sz, _vp, _i32, _i32, _i32, _vp, _vp]),
    "pa_bm_create": (_vp, [_i32, _i32, _pi32]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add_seq": (_i32, [_vp, _i64]),
    "pa_bm_append": (_i32, [_vp, _i64, _i32, _pi64]),
    "pa_bm_append_batch": (_i32, [_vp, _pi64, _i32, _pi64]),
    "pa_bm_fork": (_i32, [_vp, _i64, _i64]),
    "pa_bm_free_seq": (_i32, [_vp, _i64]),
    "pa_bm_table": (_i32, [_vp, _i64, _pi32, _i32]),
    "pa_bm_tables": (_i32, [_vp, _pi64, _i32, _pi32, _i32, _c.c_int32]),
    "pa_bm_num_tokens": (_i32, [_vp, _i64]),
    "pa_bm_num_pending_copies": (_i32, [_vp]),
    "pa_bm_take_copies": (_i32, [_vp, _pi32, _i32]),
    "pa_bm_num_free": (_i32, [_vp]),
    "pa_bm_refcount": (_i32, [_vp, _c.c_int32]),
    "pa_bm_set_host_blocks": (_i32, [_vp, _i32]),
    "pa_bm_swap_out": (_i32, [_vp, _pi64, _i32, _pi32, _i32, _c.POINTER(_c.c_int)]),
    "pa_bm_swap_in": (_i32, [_vp, _pi64, _i32, _pi32, _i32, _c.POINTER(_c.c_int)]),
    "pa_bm_is_swapped": (_i32, [_vp, _i64]),
    "pa_bm_num_host_free": (_i32, [_vp]),
    "pa_bm_host_refcount": (_i32, [_vp, _c.c_int32]),
    "pa_bm_create_cached": (_vp, [_i32, _i32, _pi32]),
    "pa_bm_add_seq_cached": (_i32, [_vp, _i64, _pi32, _i32, _c.c_char_p, _i32, _c.POINTER(_c.c_int)]),
    "pa_bm_append_tokens": (_i32, [_vp, _i64, _pi32, _i32, _pi64]),
    "pa_bm_num_cached_blocks": (_i32, [_vp]),
    "pa_bm_block_hash": (_i32, [_vp, _i64, _i32, _c.c_char_p]),
    "pa_bm_cached_block": (_i32, [_vp, _c.c_char_p]),
}


def load(path: str = LIB_PATH):
    # torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading it
    # first makes libpa's libamdhip64.so.7 dependency bind to that same copy,
    # so tensors and launches share one runtime and one device context.
    import torch  # noqa: F401

    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m paged_kv_cache_117_amd.build_lib` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = load()
