"""Pins for the oracle's cache write and block copy (CPU only)."""

import numpy as np

import oracle
from oracle.attention import gather_sequence


def test_write_lands_at_block_and_offset_of_request_a():
    """Request A (blocks 7, 1, 3) writes its 37th token at block 3, offset 4.

    PagedAttention and vLLM: Paging the KV Cache Like an OS, "Step 3": tokens
    33..37 sit in block 3, so position 36 is slot 4 of block 3.
    """
    nb, hkv, bs, d = 8, 2, 16, 4
    k = np.zeros((nb, hkv, bs, d), np.float32)
    v = np.zeros_like(k)
    kn = np.arange(1, 1 + hkv * d, dtype=np.float32).reshape(1, hkv, d)
    vn = -kn
    slot = 3 * 16 + 4
    k2, v2 = oracle.write_kv(k, v, kn, vn, [slot], bs)
    expect_k = np.zeros_like(k)
    expect_k[3, 0, 4] = [1, 2, 3, 4]
    expect_k[3, 1, 4] = [5, 6, 7, 8]
    assert np.array_equal(k2, expect_k)
    assert np.array_equal(v2, -expect_k)
    assert np.all(k == 0)  # inputs untouched


def test_write_skips_negative_slots_and_round_trips_through_gather():
    rng = np.random.default_rng(0)
    nb, hkv, bs, d = 6, 3, 16, 8
    k = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    v = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    kn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = [2 * 16 + 15, -1, 5 * 16 + 0]
    k2, v2 = oracle.write_kv(k, v, kn, vn, slots, bs)
    changed = np.argwhere(np.any(k2 != k, axis=-1))
    assert sorted(map(tuple, changed.tolist())) == sorted(
        [(2, h, 15) for h in range(hkv)] + [(5, h, 0) for h in range(hkv)])
    # a sequence whose table is [4, 2] and length 32 sees token 0's K at position 31
    seq = gather_sequence(k2, np.array([4, 2]), 32, "fp32")
    assert np.array_equal(seq[:, 31], kn[0].astype(np.float64))
    seqv = gather_sequence(v2, np.array([5]), 1, "fp32")
    assert np.array_equal(seqv[:, 0], vn[2].astype(np.float64))


def test_copy_blocks_small_example():
    k = np.arange(4 * 1 * 2 * 2, dtype=np.float32).reshape(4, 1, 2, 2)
    v = 100 + k
    k2, v2 = oracle.copy_blocks(k, v, [(0, 3), (2, 1)])
    expect = np.array(
        [[[[0, 1], [2, 3]]], [[[8, 9], [10, 11]]], [[[8, 9], [10, 11]]], [[[0, 1], [2, 3]]]],
        dtype=np.float32)
    assert np.array_equal(k2, expect)
    assert np.array_equal(v2, 100 + expect)
    assert np.array_equal(k, np.arange(16, dtype=np.float32).reshape(4, 1, 2, 2))


def test_copy_blocks_whole_block_all_heads_bitwise():
    rng = np.random.default_rng(1)
    k = rng.integers(0, 1 << 16, size=(10, 4, 16, 8), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(10, 4, 16, 8), dtype=np.uint16)
    pairs = [(1, 7), (1, 8), (4, 9)]
    k2, v2 = oracle.copy_blocks(k, v, pairs)
    for s, dd in pairs:
        assert np.array_equal(k2[dd], k[s]) and np.array_equal(v2[dd], v[s])
    untouched = [b for b in range(10) if b not in (7, 8, 9)]
    assert np.array_equal(k2[untouched], k[untouched])
    assert np.array_equal(v2[untouched], v[untouched])


def test_swap_matches_fancy_indexing_and_skips_bad_ids():
    rng = np.random.default_rng(4)
    src_k = rng.standard_normal((10, 2, 16, 8))
    src_v = rng.standard_normal((10, 2, 16, 8))
    dst_k = np.zeros((6, 2, 16, 8))
    dst_v = np.zeros((6, 2, 16, 8))
    pairs = np.array([[3, 0], [9, 5], [0, 2], [12, 1], [4, -1]])  # last two skipped
    k, v = oracle.swap_blocks(dst_k, dst_v, src_k, src_v, pairs)
    want_k = dst_k.copy()
    want_v = dst_v.copy()
    want_k[[0, 5, 2]] = src_k[[3, 9, 0]]
    want_v[[0, 5, 2]] = src_v[[3, 9, 0]]
    assert np.array_equal(k, want_k) and np.array_equal(v, want_v)
    assert np.all(dst_k == 0)  # inputs untouched


def test_swap_out_and_back_to_other_blocks_keeps_attention():
    """Preemption by swapping (PagedAttention: Virtual Memory for the KV Cache,
    "Scheduling and preemption"): a sequence's blocks go to a host pool and
    come back into different device blocks; with its table repointed, its
    attention output is unchanged, bit for bit."""
    rng = np.random.default_rng(5)
    nb, hkv, d, L = 12, 2, 16, 45
    k = rng.standard_normal((nb, hkv, 16, d))
    v = rng.standard_normal((nb, hkv, 16, d))
    table = np.array([[7, 2, 9]], np.int32)
    q = rng.standard_normal((1, 4, d))
    before = oracle.decode(q, k, v, table, [L], 0.25, "fp32")
    host_k = np.full((5, hkv, 16, d), np.nan)
    host_v = np.full_like(host_k, np.nan)
    out_pairs = [(7, 4), (2, 0), (9, 3)]
    host_k, host_v = oracle.swap_blocks(host_k, host_v, k, v, out_pairs)
    k[[7, 2, 9]] = np.nan  # the device blocks are reused meanwhile
    v[[7, 2, 9]] = np.nan
    in_pairs = [(4, 1), (0, 10), (3, 5)]
    k, v = oracle.swap_blocks(k, v, host_k, host_v, in_pairs)
    after = oracle.decode(q, k, v, np.array([[1, 10, 5]], np.int32), [L], 0.25, "fp32")
    assert np.array_equal(before, after)
