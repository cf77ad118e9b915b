"""Byte and flop counts for the decode and chunked-prefill steps (pure arithmetic, no device code).

KV bytes per token across the model: 2 (K and V) x layers x KV heads x head
dim x bytes per element (vLLM's PagedAttention: How Memory Management
Supports Large Model Inference, "2.1"; Batching and PagedAttention, "Quick
Reference", bytes per block).  The decode metric counts one layer: every
valid token's K and V row once per KV head.
"""

from __future__ import annotations

ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def block_bytes(block_size: int, num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return block_size * kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes)


def decode_kv_bytes(context_lens, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Algorithmic K+V bytes one decode launch must read (one layer)."""
    return int(sum(int(L) for L in context_lens)) * kv_bytes_per_token(1, num_kv_heads, head_dim, elem_bytes)


def decode_unique_kv_bytes(block_tables, context_lens, num_kv_heads: int, head_dim: int, elem_bytes: int,
                           block_size: int = 16) -> int:
    """K+V bytes of the distinct physical blocks one decode launch reads: a
    block shared by several sequences (a shared prefix) counts once, with
    the most slots any of them reads from it."""
    import numpy as np

    slots = {}
    tables = np.asarray(block_tables)
    for s, L in enumerate(context_lens):
        L = int(L)
        nb = -(-L // block_size)
        for j in range(nb):
            b = int(tables[s, j])
            n = min(block_size, L - j * block_size)
            if n > slots.get(b, 0):
                slots[b] = n
    return sum(slots.values()) * kv_bytes_per_token(1, num_kv_heads, head_dim, elem_bytes)


def decode_io_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    elem_bytes: int, block_size: int = 16) -> int:
    """KV bytes plus q read, out written, table entries and lengths read."""
    B = len(context_lens)
    table = sum(4 * (-(-int(L) // block_size)) for L in context_lens)
    return (decode_kv_bytes(context_lens, num_kv_heads, head_dim, elem_bytes)
            + 2 * B * num_q_heads * head_dim * elem_bytes + table + 4 * B)


def write_kv_bytes(num_tokens: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """New K/V rows read and written, plus the int64 slots."""
    return num_tokens * (2 * 2 * num_kv_heads * head_dim * elem_bytes + 8)


def prefill_pairs(prior_lens, chunk_lens) -> int:
    """(query token, key position) pairs of one chunked-prefill launch per
    query head: token i of a chunk of T after P cached tokens sees P + i + 1
    positions."""
    n = 0
    for P, T in zip(prior_lens, chunk_lens):
        P, T = int(P), int(T)
        n += T * P + T * (T + 1) // 2
    return n


def prefill_flops(prior_lens, chunk_lens, num_q_heads: int, head_dim: int) -> int:
    """Algorithmic flops of one chunked-prefill attention launch: per (query
    head, query token, visible position) 2*D for the score and 2*D for the
    weighted V row (the softmax itself is not counted)."""
    return 4 * head_dim * num_q_heads * prefill_pairs(prior_lens, chunk_lens)


def prefill_io_bytes(prior_lens, chunk_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     elem_bytes: int) -> int:
    """Each sequence's K+V rows read once, q read and out written once."""
    ctx = sum(int(P) + int(T) for P, T in zip(prior_lens, chunk_lens))
    toks = sum(int(T) for T in chunk_lens)
    return (ctx * kv_bytes_per_token(1, num_kv_heads, head_dim, elem_bytes)
            + 2 * toks * num_q_heads * head_dim * elem_bytes)


def write_decode_io_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          elem_bytes: int, block_size: int = 16) -> int:
    """pa_write_kv_decode: decode_io_bytes plus each sequence's new K and V
    rows read from k_new / v_new and written into the pool."""
    B = len(context_lens)
    return (decode_io_bytes(context_lens, num_q_heads, num_kv_heads, head_dim, elem_bytes, block_size)
            + B * 2 * 2 * num_kv_heads * head_dim * elem_bytes)
