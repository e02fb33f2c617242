"""Worked examples printed on the pages (tests/golden/*.json, each with its
citation) against the block manager, the slot arithmetic and the byte
accounting (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle
from workloads import BlockManager, OutOfPages
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["page_table_figure.json", "flowchart_block_table.json"])
def test_block_table_figures(name):
    fig = load(name)
    bs, pages, n = fig["block_size"], fig["pages"], fig["num_tokens"]
    assert len(pages) == -(-n // bs)
    for i, (lo, hi) in enumerate(fig["block_ranges"]):
        for t in (lo, hi):
            assert oracle.resolve_slot(pages, t, bs)[0] == pages[i]
    for t, page, off in fig["probes_token_page_offset"]:
        assert oracle.resolve_slot(pages, t, bs) == (page, off)
    # a block manager whose free list starts with the figure's pages hands them out in order
    free = pages + [p for p in range(max(pages) + 1) if p not in pages]
    mgr = BlockManager(len(free), bs, free_order=free)
    assert mgr.allocate("s", n) == pages
    for t, page, off in fig["probes_token_page_offset"]:
        assert mgr.slot("s", t) == page * bs + off


def test_tiny_figure_workload_uses_figure_pages():
    fig = load("page_table_figure.json")
    w = workloads.tiny(figure_table=True)
    assert w.context_lens[0] == fig["num_tokens"]
    assert w.block_tables[0, :3].tolist() == fig["pages"]
    # the appended token (position 35) lands in page 2 at offset 3
    assert w.append_slots[0] == 2 * 16 + 3


def test_allocator_demo():
    ex = load("allocator_demo.json")
    mgr = BlockManager(ex["num_blocks"], ex["block_size"])
    pages = mgr.allocate("r", ex["num_tokens"])
    assert len(pages) == ex["pages_taken"]
    assert len(pages) * ex["block_size"] == ex["capacity_tokens"]
    assert mgr.num_free() == ex["num_blocks"] - ex["pages_taken"]


def test_block_manager_allocate_and_free():
    ex = load("block_manager_test.json")
    mgr = BlockManager(ex["total_pages"], ex["block_size"])
    pages = mgr.allocate("seq_1", ex["num_tokens"])
    assert len(pages) == ex["pages_taken"]
    assert mgr.num_free() == ex["free_after_allocate"]
    mgr.free_sequence("seq_1")
    assert mgr.num_free() == ex["free_after_free"]


def test_kv_bytes_per_token_llama3_70b():
    ex = load("kv_bytes_llama3_70b.json")
    per_token = 2 * ex["layers"] * ex["kv_heads"] * ex["head_dim"] * ex["bytes_per_element"]
    assert per_token == ex["bytes_per_token"]
    assert per_token * ex["tokens"] == ex["bytes_for_tokens"]
    # the printed "1.31 GB" is the byte count in KiB divided by 10^6
    assert round(ex["bytes_for_tokens"] / 1024 / 1e6, 2) == ex["printed_gb"]
    # one layer of the 70B-shaped workload: 2 * 8 * 128 * 2 bytes per token
    w = workloads.llama3_70b(num_seqs=4)
    assert w.kv_bytes_per_token() * ex["layers"] == ex["bytes_per_token"]


def test_internal_fragmentation_example():
    ex = load("internal_fragmentation.json")
    waste = 1 - ex["used_tokens"] / ex["reserved_tokens"]
    assert waste == ex["waste_fraction"]
    assert round(ex["printed_reserved_gb"] * waste, 2) == ex["printed_waste_gb"]


def test_exhaustion_raises_memory_error():
    mgr = BlockManager(2, 16)
    with pytest.raises(MemoryError):
        mgr.allocate("a", 33)
    mgr.allocate("a", 32)
    with pytest.raises(OutOfPages):
        mgr.append_token("a")               # token 32 opens a third block
    assert mgr.lengths["a"] == 32


def test_append_trigger_takes_a_page_when_a_block_opens():
    bs = 16
    mgr = BlockManager(8, bs)
    mgr.allocate("s", 1)
    taken = []
    for _ in range(40):
        before = len(mgr.tables["s"])
        mgr.append_token("s")
        count = mgr.lengths["s"]
        if len(mgr.tables["s"]) != before:
            taken.append(count)
    # the listing's trigger: count % bs == 1 with count = length after the token
    assert taken == [c for c in range(2, 42) if c % bs == 1] == [17, 33]
