"""CPU oracle for the paged decode step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``paged_kv_cache_117_amd``
and its HIP library) never imports, links or calls anything here, and nothing
here imports the product.  The only code both sides share is the seeded input
generator in ``workloads/``, which holds none of the method's arithmetic.

What it computes, each part written as the plain definition from the pages:

* ``attention.decode`` -- for every sequence, gather its K/V rows through its
  block table into contiguous arrays, then exact two-pass softmax attention in
  float64 (PagedAttention and vLLM: Paging the KV Cache Like an OS, "Step 5:
  attention over scattered blocks"; PagedAttention (tensortonic), "5. Reading
  the Cache During Attention"; PagedAttention: Virtual Memory for the KV Cache,
  "PagedAttention: attention over non-contiguous blocks").
* ``attention.prefill`` -- several new tokens per sequence (a prefill
  chunk): token i of the T new ones sits at position L - T + i and attends
  causally to positions 0..L-T+i, same two-pass float64 softmax (Batching and
  PagedAttention, chunked prefill; vLLM's PagedAttention: How Memory
  Management Supports Large Model Inference, "2.5").
* ``cache_ops.write_kv`` -- store each new token's K/V at its block+offset
  (PagedAttention (tensortonic), "5. Reading the Cache During Attention";
  Paging the KV Cache Like an OS, "Step 5", the write kernel).
* ``cache_ops.copy_blocks`` -- whole-block copies for copy-on-write (Paging
  the KV Cache Like an OS, "Step 4" and the copy kernel of "Step 5").
* ``cache_ops.swap_blocks`` -- whole blocks between the device pool and a
  host pool, out and back, for preemption by swapping (PagedAttention:
  Virtual Memory for the KV Cache, "Scheduling and preemption").
* ``block_manager.BlockManager`` -- free list, reference counts, on-demand
  allocation, fork and copy-on-write (Paging the KV Cache Like an OS, "Step 3"
  and "Step 4"; PagedAttention (tensortonic), "7. Sharing a Prefix Without
  Overwriting It"; Batching and PagedAttention, "How on-demand allocation
  eliminates waste").

Pins (see ``tests/test_oracle*.py``): brute-force contiguous attention from a
library routine (torch's scaled_dot_product_attention in float64), closed-form
special cases, placement invariance, shared-vs-duplicated prefixes, the
partition-merge identity, and the pages' worked examples for the block
manager.  Every function here is pinned; none is "parity unpinned".
"""

from . import attention, block_manager, cache_ops  # noqa: F401
from .attention import decode, prefill, storage_to_f64  # noqa: F401
from .block_manager import BlockManager, NoFreeBlocks  # noqa: F401
from .cache_ops import copy_blocks, swap_blocks, write_kv  # noqa: F401
