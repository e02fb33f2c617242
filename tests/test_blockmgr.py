"""Host block manager: FIFO reuse, reference counts, forks and copy-on-write."""

import numpy as np
import pytest

from workloads import BlockManager


def test_fifo_reuse_order():
    mgr = BlockManager(6, 16, free_order=[5, 4, 3, 2, 1, 0])
    assert mgr.allocate("a", 20) == [5, 4]
    assert mgr.allocate("b", 1) == [3]
    mgr.free_sequence("a")
    assert list(mgr.free) == [2, 1, 0, 5, 4]
    assert mgr.allocate("c", 48) == [2, 1, 0]


def test_fork_shares_and_free_respects_refcounts():
    mgr = BlockManager(8, 16)
    mgr.allocate("p", 40)               # pages 0, 1, 2
    mgr.fork("p", "c")
    assert mgr.tables["c"] == [0, 1, 2] and mgr.ref[:3] == [2, 2, 2]
    mgr.free_sequence("p")
    assert mgr.num_free() == 5 and mgr.ref[:3] == [1, 1, 1]
    mgr.free_sequence("c")
    assert mgr.num_free() == 8


def test_copy_on_write_only_while_shared():
    bs = 16
    mgr = BlockManager(10, bs)
    mgr.allocate("p", 20)               # pages 0, 1; page 1 holds 4 tokens
    mgr.fork("p", "a")
    mgr.fork("p", "b")
    s = mgr.append_token("a")           # writes into shared page 1 -> copy to page 2
    assert mgr.take_copies() == [(1, 2)]
    assert mgr.tables["a"] == [0, 2] and s == 2 * bs + 4
    s = mgr.append_token("b")           # page 1 still shared with p -> copy to page 3
    assert mgr.take_copies() == [(1, 3)] and s == 3 * bs + 4
    s = mgr.append_token("p")           # p is the last holder of page 1: in place
    assert mgr.take_copies() == [] and s == 1 * bs + 4
    assert mgr.ref[:4] == [3, 1, 1, 1]


def test_new_block_after_fork_needs_no_copy():
    mgr = BlockManager(6, 16)
    mgr.allocate("p", 32)
    mgr.fork("p", "c")
    mgr.append_token("c")               # token 32 opens a new block: fresh page, no copy
    assert mgr.take_copies() == []
    assert mgr.tables["c"] == [0, 1, 2] and mgr.tables["p"] == [0, 1]


def test_invalid_arguments():
    with pytest.raises(ValueError):
        BlockManager(3, 16, free_order=[0, 0, 1])
    mgr = BlockManager(3, 16)
    mgr.allocate("a", 3)
    with pytest.raises(KeyError):
        mgr.allocate("a", 3)
    with pytest.raises(IndexError):
        mgr.slot("a", 3)
