"""Block-manager behaviour pinned by the pages' worked examples and invariants.

Written against a small interface that both the oracle block manager and the
library's C++ block manager (through its Python binding) implement:
``add_seq, append(seq, n) -> slots, append_batch(seqs) -> slots, fork,
free_seq, take_copies() -> [(src, dst)], table, num_tokens, num_free,
refcount``.  ``make(num_blocks, block_size, free_order)`` builds one and
``no_blocks`` is the exception it raises when the pool runs dry.
"""

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def used_blocks(bm, n):
    return sum(1 for b in range(n) if bm.refcount(b) > 0)


def check_request_a(make, no_blocks):
    g = golden()["request_a"]
    n = 64
    order = g["blocks"] + [b for b in range(n) if b not in g["blocks"]]
    bm = make(n, g["block_size"], order)
    bm.add_seq(0)
    slots = bm.append(0, g["prompt"])
    assert bm.table(0) == g["blocks"]
    assert len(bm.table(0)) * 16 - g["prompt"] == g["empty_after_prefill"]
    assert slots[-1] == 3 * 16 + 4  # token 37 -> block 3, offset 4
    bm.append(0, g["decode_steps"])
    assert bm.num_tokens(0) == g["tokens_after_decode"]
    assert len(bm.table(0)) * 16 - bm.num_tokens(0) == g["free_after_decode"]
    bm.append(0, g["last_token_fitting_three_blocks"] - g["tokens_after_decode"])
    assert len(bm.table(0)) == 3
    bm.append(0, 1)
    assert bm.num_tokens(0) == g["first_token_needing_fourth_block"]
    assert len(bm.table(0)) == 4 and bm.table(0)[3] == order[3]
    bm.free_seq(0)
    assert bm.num_free() == n


def check_paged_rerun(make, no_blocks):
    g = golden()
    reqs = g["reservation_example"]["requests_prompt_generated_final"]
    r = g["paged_rerun"]
    n = 400
    bm = make(n, 16, None)
    used = 0
    for i, (p, gen, _) in enumerate(reqs):
        bm.add_seq(i)
        bm.append(i, p + gen)
        used += p + gen
    blocks = n - bm.num_free()
    assert blocks == r["blocks"]
    assert round(used / (blocks * 16), 4) == r["utilisation"]
    kib = g["reservation_example"]["kib_per_token"]
    assert blocks * 16 * kib / 1024 == r["mib"]
    assert g["reservation_example"]["reserved_mib"] - r["mib"] == r["freed_mib"]


def check_parallel_sampling(make, no_blocks):
    g = golden()["parallel_sampling"]
    n = 1000
    bm = make(n, g["block_size"], None)
    bm.add_seq(0)
    bm.append(0, g["prompt"])
    for c in range(1, g["samples"]):
        bm.fork(0, c)
    for c in range(g["samples"]):
        bm.append(c, g["generated"])
    pairs = bm.take_copies()
    in_use = n - bm.num_free()
    assert in_use == g["blocks_with_sharing"]
    assert in_use * 2 == g["mib_with_sharing"]  # 2 MiB per Llama-3.1-8B block
    # the first n-1 writers copy the partial 63rd block; the last writes in place
    assert len(pairs) == g["samples"] - 1
    shared = bm.table(0)[: g["shared_full_prompt_blocks"]]
    for c in range(g["samples"]):
        t = bm.table(c)
        assert t[: g["shared_full_prompt_blocks"]] == shared
        assert len(t) - g["shared_full_prompt_blocks"] == g["private_blocks_per_sample"]
    for b in shared:
        assert bm.refcount(b) == g["samples"]
    # without sharing
    bm2 = make(n, g["block_size"], None)
    for c in range(g["samples"]):
        bm2.add_seq(c)
        bm2.append(c, g["prompt"] + g["generated"])
    assert n - bm2.num_free() == g["blocks_without_sharing"]
    assert (n - bm2.num_free()) * 2 == g["mib_without_sharing"]
    assert round(100 * (1 - in_use / (n - bm2.num_free()))) == g["pct_less"]


def check_four_token_blocks(make, no_blocks):
    g = golden()["four_token_blocks"]
    order = g["table_example"] + [b for b in range(8) if b not in g["table_example"]]
    bm = make(8, g["block_size"], order)
    bm.add_seq(0)
    bm.append(0, 6)
    assert len(bm.table(0)) == g["six_tokens_blocks"]
    assert len(bm.table(0)) * 4 - 6 == g["six_tokens_left_over"]
    bm.append(0, 2)
    assert len(bm.table(0)) == g["eight_tokens_blocks"]
    bm.append(0, 1)
    assert len(bm.table(0)) == g["nine_tokens_blocks"]
    assert len(bm.table(0)) * 4 == g["nine_tokens_capacity"]
    assert g["nine_tokens_capacity"] - 9 == g["nine_tokens_unused"]
    assert bm.table(0) == g["table_example"]


def check_prefix_cow(make, no_blocks):
    g = golden()["prefix_cow"]
    bm = make(8, g["block_size"], None)
    bm.add_seq(0)  # A
    bm.append(0, 6)  # blocks [full 4][2 of 4]
    first, second = bm.table(0)
    bm.fork(0, 1)  # B
    bm.append(1, 1)  # B writes into the shared partial block -> copy
    pairs = bm.take_copies()
    assert pairs == [(second, bm.table(1)[1])]
    assert len(pairs) == g["copied_blocks_for_b"]
    assert bm.table(1)[0] == first  # the first four entries stay shared
    assert bm.refcount(first) == 2
    bm.free_seq(0)  # A finishes
    assert bm.refcount(first) == 1  # B still holds it: not reclaimed
    assert bm.refcount(second) == 0
    assert bm.num_free() == 8 - 2


def check_test_yourself(make, no_blocks):
    g = golden()["test_yourself"]
    bm = make(g["pool_blocks"], g["block_size"], None)
    for i in range(g["short_requests"]):
        bm.add_seq(i)
        bm.append(i, g["short_prompt"] + g["short_generated"])
    assert len(bm.table(0)) == g["short_blocks_each"]
    assert g["pool_blocks"] - bm.num_free() == g["short_blocks"]
    for i in range(g["long_requests"]):
        bm.add_seq(1000 + i)
        bm.append(1000 + i, g["long_prompt"])
    assert len(bm.table(1000)) == g["long_blocks_each"]
    assert g["pool_blocks"] - bm.num_free() == g["total_blocks"]
    for i in range(g["long_requests"]):
        bm.append(1000 + i, 100)
    assert g["pool_blocks"] - bm.num_free() == g["total_after_long_generate_100"]
    assert g["static_reservation"] - (g["short_prompt"] + g["short_generated"]) == g["static_unused_per_short"]


def check_waste_bound(make, no_blocks):
    g = golden()["short_sequence_waste"]
    bm = make(64, 16, None)
    bm.add_seq(0)
    for L in range(1, 700):
        bm.append(0, 1)
        nb = len(bm.table(0))
        assert nb == math.ceil(L / 16)
        assert 0 <= nb * 16 - L <= g["max_wasted_slots"]
    assert g["max_wasted_slots"] / g["tokens"] * 100 < g["max_overhead_pct"]


def snapshot(bm, n, seqs):
    return (
        bm.num_free(),
        [bm.refcount(b) for b in range(n)],
        {s: (bm.table(s), bm.num_tokens(s)) for s in seqs},
    )


def check_all_or_nothing(make, no_blocks):
    bm = make(5, 16, None)
    bm.add_seq(0)
    bm.append(0, 40)  # 3 blocks
    bm.fork(0, 1)
    before = snapshot(bm, 5, [0, 1])
    try:
        bm.append(1, 60)  # COW + 3 new blocks > 2 free
        raise AssertionError("expected the pool to run dry")
    except no_blocks:
        pass
    assert snapshot(bm, 5, [0, 1]) == before
    assert bm.take_copies() == []
    bm.add_seq(2)
    bm.append(2, 17)  # takes the last 2 blocks
    before = snapshot(bm, 5, [0, 1, 2])
    try:
        bm.append_batch([0, 1, 2])  # 0 and 1 need copies
        raise AssertionError("expected the pool to run dry")
    except no_blocks:
        pass
    assert snapshot(bm, 5, [0, 1, 2]) == before
    bm.free_seq(2)
    slots = bm.append_batch([0, 1])  # first copies, second finds count 1
    assert len(slots) == 2
    assert len(bm.take_copies()) == 1


def check_random_invariants(make, no_blocks, seed=0, n=48, bs=4, steps=2000):
    rng = np.random.default_rng(seed)
    bm = make(n, bs, rng.permutation(n).tolist())
    live = []
    nxt = 0
    pend = 0
    for _ in range(steps):
        op = rng.integers(0, 6)
        if op == 0 or not live:
            bm.add_seq(nxt)
            live.append(nxt)
            nxt += 1
        elif op == 1 or op == 2:
            s = live[rng.integers(len(live))]
            try:
                bm.append(s, int(rng.integers(0, 9)))
            except no_blocks:
                pass
        elif op == 3:
            s = live[rng.integers(len(live))]
            bm.fork(s, nxt)
            live.append(nxt)
            nxt += 1
        elif op == 4:
            s = live.pop(rng.integers(len(live)))
            bm.free_seq(s)
        else:
            pend += len(bm.take_copies())
        refs = [bm.refcount(b) for b in range(n)]
        assert sum(refs) == sum(len(bm.table(s)) for s in live)
        for s in live:
            assert len(bm.table(s)) == -(-bm.num_tokens(s) // bs)
        assert bm.num_free() <= n - sum(1 for r in refs if r > 0)
    for s in live:
        bm.free_seq(s)
    bm.take_copies()
    assert bm.num_free() == n
    assert all(bm.refcount(b) == 0 for b in range(n))


ALL_CHECKS = [
    check_request_a,
    check_paged_rerun,
    check_parallel_sampling,
    check_four_token_blocks,
    check_prefix_cow,
    check_test_yourself,
    check_waste_bound,
    check_all_or_nothing,
    check_random_invariants,
]
