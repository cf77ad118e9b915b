"""Oracle: single-query decode attention read through block tables, fp64.

Definition followed (plain attention; paging changes only the addresses):

* PagedAttention: Virtual Memory for the KV Cache, "PagedAttention: attention
  over non-contiguous blocks" -- the block-wise softmax: the query is scored
  against the keys of every logical block, exponentiated, normalised by the
  sum over all blocks up to the query's position, and the weights combine the
  value rows.  The transcription on that page is garbled (a ones-vector sits
  inside the exponent, and the sums run over whole blocks); it is read here as
  the ordinary softmax over the valid positions 0..L-1 only, with the last
  block truncated at the context length.
* PagedAttention (tensortonic), "5. Reading the Cache During Attention" --
  the query attends to the valid keys and values of its sequence, including
  the current position; the sequence length marks which slots of the final
  block are valid; softmax normalises over all valid positions at once.
* PagedAttention and vLLM: Paging the KV Cache Like an OS, "Step 3: blocks
  and block tables" -- logical block j holds positions 16j..16j+15; the table
  maps it to a physical block.
* Grouped-query attention (vLLM's PagedAttention: How Memory Management
  Supports Large Model Inference, "2.1"): several query heads share one KV
  head.  The pages do not state which; query head h reads KV head h // g with
  g = num_q_heads / num_kv_heads (contiguous groups).

Steps, in order: gather -> scores -> max -> exp -> sum -> weighted sum of V.
"""

from __future__ import annotations

import numpy as np


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored fp32 / fp16 / bf16-bits values to float64."""
    if dtype in ("fp32", "fp16"):
        return np.asarray(a).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def gather_sequence(pool: np.ndarray, table_row: np.ndarray, L: int, dtype: str) -> np.ndarray:
    """Contiguous [num_kv_heads][L][head_dim] float64 copy of one sequence.

    Position t lives in physical block ``table_row[t // bs]`` at slot
    ``t % bs``.  Only the first ceil(L/bs) table entries are read.
    """
    _, hkv, bs, d = pool.shape
    out = np.empty((hkv, L, d), dtype=np.float64)
    for t in range(0, L, bs):
        phys = int(table_row[t // bs])
        n = min(bs, L - t)
        out[:, t:t + n, :] = storage_to_f64(pool[phys, :, :n, :], dtype)
    return out


def decode(q, k_pool, v_pool, block_tables, context_lens, scale, dtype: str) -> np.ndarray:
    """Paged decode attention, float64.

    q            [B][Hq][D] storage values
    k_pool/v_pool[num_blocks][Hkv][bs][D] storage values
    block_tables [B][max_blocks] int (entries past ceil(L/bs) are never read)
    context_lens [B] int (L = 0 gives a zero row)
    scale        the fp32 scale, used as its exact float64 value
    returns      [B][Hq][D] float64
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    assert Hq % Hkv == 0
    g = Hq // Hkv
    sc = np.float64(np.float32(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            continue
        K = gather_sequence(k_pool, block_tables[s], L, dtype)
        V = gather_sequence(v_pool, block_tables[s], L, dtype)
        qs = storage_to_f64(q[s], dtype)
        for h in range(Hq):
            j = h // g
            x = sc * (K[j] @ qs[h])  # scores over the L valid positions
            m = x.max()
            w = np.exp(x - m)
            out[s, h] = (w / w.sum()) @ V[j]
    return out


def prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, dtype: str) -> np.ndarray:
    """Paged attention for several new tokens per sequence (chunked prefill), float64.

    Definition followed:

    * Batching and PagedAttention, "How continuous batching keeps the GPU
      saturated" and its FAQ on chunked prefill -- a long prompt is fed over
      several steps, a chunk of consecutive tokens per step, each chunk filling
      blocks of the paged cache.
    * vLLM's PagedAttention: How Memory Management Supports Large Model
      Inference, "2.5" -- a request keeps the count of tokens already computed
      and each step computes the next run of tokens, which covers chunked
      prefill and continuing after a prefix-cache hit alike.
    * PagedAttention (tensortonic), "5. Reading the Cache During Attention" --
      where a token sits in memory changes neither its logical position nor
      the causal mask; softmax normalises over every position the query may
      see.

    Reading (the pages give no formula for several query tokens): sequence s
    has ``L = context_lens[s]`` cached positions, of which the last
    ``T = query_start[s+1] - query_start[s]`` are this step's tokens, already
    written to the pool.  Its i-th new token sits at position ``p = L - T + i``
    and attends, causally, to positions ``0..p``.  Query heads map to KV heads
    as in :func:`decode`.

    q            [N][Hq][D] storage values, N = query_start[-1]; rows of
                 sequence s are query_start[s] .. query_start[s+1]-1
    k_pool/v_pool[num_blocks][Hkv][bs][D] storage values
    block_tables [B][max_blocks] int
    context_lens [B] int, each >= that sequence's T
    query_start  [B+1] int, non-decreasing, query_start[0] = 0
    scale        the fp32 scale, used as its exact float64 value
    returns      [N][Hq][D] float64
    """
    q = np.asarray(q)
    N, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    assert Hq % Hkv == 0
    g = Hq // Hkv
    qs = [int(x) for x in query_start]
    assert qs[0] == 0 and qs[-1] == N
    sc = np.float64(np.float32(scale))
    out = np.zeros((N, Hq, D), dtype=np.float64)
    for s in range(len(qs) - 1):
        T = qs[s + 1] - qs[s]
        L = int(context_lens[s])
        assert 0 <= T <= L
        if T == 0:
            continue
        K = gather_sequence(k_pool, block_tables[s], L, dtype)
        V = gather_sequence(v_pool, block_tables[s], L, dtype)
        qf = storage_to_f64(q[qs[s]:qs[s + 1]], dtype)
        for i in range(T):
            p = L - T + i  # position of this token; it sees 0..p
            for h in range(Hq):
                j = h // g
                x = sc * (K[j, :p + 1] @ qf[i, h])
                m = x.max()
                w = np.exp(x - m)
                out[qs[s] + i, h] = (w / w.sum()) @ V[j, :p + 1]
    return out
