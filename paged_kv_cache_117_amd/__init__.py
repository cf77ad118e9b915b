"""Paged KV cache decode and chunked-prefill path for AMD MI355X (gfx950).

The device work runs in hand-written HIP kernels inside ``libpa.so`` (C ABI in
``include/pa.h``); this package only marshals arguments.  Importing it loads
the library and fails with ImportError when it has not been built.

    decode(q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len)
    prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, max_query_len, max_context_len)
    write_kv(k_pool, v_pool, k_new, v_new, slot_mapping)
    write_kv_decode(q, k_pool, v_pool, k_new, v_new, block_tables, context_lens, scale, max_context_len)
    copy_blocks(k_pool, v_pool, block_pairs)
    swap_blocks(dst_k, dst_v, src_k, src_v, block_pairs)   # device <-> pinned host pool
    BlockManager(num_blocks, block_size=16, free_order=None)
"""

from ._lib import LIB, LIB_PATH  # noqa: F401  (raises ImportError if libpa.so is missing)
from .block_manager import BlockManager  # noqa: F401
from .ops import (  # noqa: F401
    NoFreeBlocks,
    PaError,
    abi_version,
    copy_blocks,
    decode,
    decode_workspace_bytes,
    prefill,
    prefill_workspace_bytes,
    probe_read,
    swap_blocks,
    time_next_main_kernel,
    write_kv,
    write_kv_decode,
)
