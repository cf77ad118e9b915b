"""Oracle: the cache write (reshape-and-cache) and copy-on-write block copies.

* ``write_kv`` -- PagedAttention (tensortonic), "5. Reading the Cache During
  Attention": the new token's key and value are written to the block and
  offset the cache manager assigned.  A slot names (block, offset) as
  ``block * block_size + offset``; negative slots are skipped.
* ``copy_blocks`` -- PagedAttention and vLLM: Paging the KV Cache Like an OS,
  "Step 4" (copy-on-write copies the block's tokens into a fresh block) and
  "Step 5" (one kernel batches many small block copies).  The whole block is
  copied: every KV head, every slot.

* ``swap_blocks`` -- PagedAttention: Virtual Memory for the KV Cache,
  "Scheduling and preemption": an evicted sequence's blocks are copied to
  CPU memory and brought back later.  Whole blocks again, from one pool to
  another pool of the same block shape (the block ids may differ).

All return new arrays and leave the inputs untouched.
"""

from __future__ import annotations

import numpy as np


def write_kv(k_pool, v_pool, k_new, v_new, slot_mapping, block_size: int):
    """k_pool/v_pool [num_blocks][Hkv][bs][D]; k_new/v_new [T][Hkv][D]."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        k[block, :, offset, :] = k_new[i]
        v[block, :, offset, :] = v_new[i]
    return k, v


def copy_blocks(k_pool, v_pool, pairs):
    """pairs: iterable of (src, dst) physical block ids."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        k[dst] = k[src]
        v[dst] = v[src]
    return k, v


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs):
    """dst[d] = src[s] for every (s, d) in pairs; ids outside a pool are skipped."""
    k = np.array(dst_k, copy=True)
    v = np.array(dst_v, copy=True)
    ns, nd = len(src_k), len(dst_k)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        if 0 <= src < ns and 0 <= dst < nd:
            k[dst] = src_k[src]
            v[dst] = src_v[src]
    return k, v
