"""Pins for the oracle block manager: the pages' worked examples and invariants."""

import pytest

import oracle
from bm_cases import ALL_CHECKS


def make_oracle(n, bs, order):
    return oracle.BlockManager(n, bs, order)


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_block_manager(check):
    check(make_oracle, oracle.NoFreeBlocks)


def test_copy_source_is_held_until_copies_are_taken():
    """A block named by a pending copy is not reused before the copy runs."""
    bm = oracle.BlockManager(4, 4, [0, 1, 2, 3])
    bm.add_seq(0)
    bm.append(0, 2)  # block 0, partial
    bm.fork(0, 1)
    bm.append(1, 1)  # copy (0 -> 1)
    bm.free_seq(0)  # block 0 reaches zero but is the pending copy's source
    assert bm.num_free() == 2 and 0 not in bm.free
    assert bm.take_copies() == [(0, 1)]
    assert list(bm.free) == [2, 3, 0]
