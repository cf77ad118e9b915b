"""Pins for the oracle's prefix cache and swapping (CPU only).

The prefix cache is checked against what the pages state: hashes chained
over the prefix (a change anywhere before a block changes its key), an extra
key that separates otherwise equal blocks, full blocks only, a full hit that
still computes its last token, freed blocks that stay reusable until the
front of the free queue reaches them (least recently freed first), and blocks
in use that are never evicted.  Swapping is checked for the group rules and
for sharing surviving a round trip.
"""

import hashlib

import pytest

from oracle.block_manager import BlockManager, NoFreeBlocks
from oracle.prefix_cache import CachingBlockManager, chain_hash

BS = 16


def test_chain_hash_is_sha256_of_the_documented_bytes():
    toks = list(range(100, 116))
    body = b"".join(t.to_bytes(4, "little") for t in toks)
    assert chain_hash(None, toks) == hashlib.sha256(bytes(32) + body).digest()
    p = hashlib.sha256(b"x").digest()
    assert chain_hash(p, toks, b"lora-7") == hashlib.sha256(p + body + b"lora-7").digest()


def _hashes(tokens, extra=b""):
    out, parent = [], None
    for j in range(len(tokens) // BS):
        parent = chain_hash(parent, tokens[j * BS:(j + 1) * BS], extra)
        out.append(parent)
    return out


def test_one_token_changes_every_later_key_and_no_earlier_one():
    a = list(range(64))
    b = list(a)
    b[20] = 999  # inside block 1
    ha, hb = _hashes(a), _hashes(b)
    assert ha[0] == hb[0]
    assert all(x != y for x, y in zip(ha[1:], hb[1:]))


def test_extra_key_separates_equal_tokens():
    t = list(range(32))
    assert _hashes(t, b"") != _hashes(t, b"adapter-1")
    assert _hashes(t, b"adapter-1") == _hashes(t, b"adapter-1")


def _fill(bm, seq, tokens, extra=b""):
    n = bm.add_seq_cached(seq, tokens, extra)
    bm.append_tokens(seq, tokens[n:])
    return n


def test_only_full_blocks_are_cached_and_a_later_request_reuses_them():
    bm = CachingBlockManager(20, BS)
    prompt = list(range(40))  # 2 full blocks + 8 tokens
    assert _fill(bm, 0, prompt) == 0
    assert bm.num_cached_blocks() == 2
    first = bm.table(0)
    # a second request with the same first 33 tokens and a different tail
    other = prompt[:33] + [7] * 10
    assert bm.add_seq_cached(1, other) == 32
    assert bm.table(1) == first[:2]
    assert bm.refcount(first[0]) == 2 and bm.refcount(first[2]) == 1


def test_full_hit_still_computes_the_last_token():
    bm = CachingBlockManager(20, BS)
    prompt = list(range(32))
    _fill(bm, 0, prompt)
    bm.free_seq(0)
    assert bm.add_seq_cached(1, prompt) == 31
    slots = bm.append_tokens(1, prompt[31:])
    assert slots == [bm.table(1)[1] * BS + 15]  # the same slot, written again in place (count 1)
    assert bm.num_tokens(1) == 32 and len(bm.pending) == 0


def test_full_hit_on_a_shared_block_copies_before_writing():
    bm = CachingBlockManager(20, BS)
    prompt = list(range(32))
    _fill(bm, 0, prompt)  # still holds the blocks
    assert bm.add_seq_cached(1, prompt) == 31
    bm.append_tokens(1, prompt[31:])
    (src, dst), = bm.take_copies()
    assert src == bm.table(0)[1] and dst == bm.table(1)[1]
    assert bm.cached_block(bm.block_hash(0, 1)) == src  # the first block keeps the entry


def test_freed_blocks_stay_cached_until_reused_least_recent_first():
    n = 8
    bm = CachingBlockManager(n, BS)
    a, b = list(range(32)), list(range(1000, 1032))
    _fill(bm, 0, a)
    _fill(bm, 1, b)
    ta, tb = bm.table(0), bm.table(1)
    bm.free_seq(0)  # freed first: evicted first
    bm.free_seq(1)
    assert bm.num_cached_blocks() == 4
    bm.add_seq(2)
    bm.append(2, 4 * BS)  # takes the 4 never-used blocks: nothing evicted
    assert bm.num_cached_blocks() == 4
    bm.append(2, BS)  # next from the front: a's last block (a's blocks went back last first)
    assert bm.table(2)[-1] == ta[1]
    assert bm.cached_block(_hashes(a)[1]) == -1 and bm.cached_block(_hashes(a)[0]) == ta[0]
    # a's first block still hits; its second no longer does
    assert bm.add_seq_cached(3, a) == 16
    assert bm.cached_block(_hashes(b)[0]) == tb[0]


def test_blocks_in_use_are_never_evicted():
    bm = CachingBlockManager(4, BS)
    a = list(range(32))
    _fill(bm, 0, a)  # holds 2 blocks, both cached
    bm.add_seq(1)
    bm.append(1, 2 * BS)
    with pytest.raises(NoFreeBlocks):
        bm.append(1, 1)
    assert bm.num_cached_blocks() == 2
    assert bm.add_seq_cached(2, a) == 31


def test_swap_round_trip_keeps_sharing_and_refuses_outside_sharing():
    bm = BlockManager(16, BS)
    bm.set_host_blocks(10)
    bm.add_seq(0)
    bm.append(0, 40)
    bm.fork(0, 1)  # shares all 3 blocks
    bm.append(1, 1)  # copy-on-write of the partial last block
    with pytest.raises(ValueError):
        bm.swap_out([0])  # a copy is pending
    bm.take_copies()
    with pytest.raises(ValueError):
        bm.swap_out([0])  # blocks 0, 1 are shared with sequence 1
    free_before = bm.num_free()
    out = bm.swap_out([0, 1])
    assert len(out) == 4  # 2 shared + 2 private last blocks, each once
    assert bm.num_free() == free_before + 4
    assert bm.table(0)[:2] == bm.table(1)[:2]  # host ids, still shared
    with pytest.raises(ValueError):
        bm.append(0, 1)
    back = bm.swap_in([0, 1])
    assert [h for h, _ in back] == [h for _, h in out]
    assert bm.table(0)[:2] == bm.table(1)[:2]
    assert bm.refcount(bm.table(0)[0]) == 2 and bm.refcount(bm.table(0)[2]) == 1


def test_swap_out_is_all_or_nothing():
    bm = BlockManager(16, BS)
    bm.set_host_blocks(2)
    bm.add_seq(0)
    bm.append(0, 40)  # 3 blocks
    t = bm.table(0)
    with pytest.raises(NoFreeBlocks):
        bm.swap_out([0])
    assert bm.table(0) == t and not bm.is_swapped(0) and len(bm.host_free) == 2
