"""The native page allocator (include/pa_blockmgr.h) on the host (CPU only).

Pinned three ways: the worked examples the pages print (tests/golden/*.json,
each with its citation); the behaviour cases of the host block manager the
workloads use; and differential runs -- random operation sequences and every
named workload at full size -- that must match that host manager bit for bit
(every page id, slot, copy pair, reference count and the free-list order)."""

import json
import os

import numpy as np
import pytest

import workloads
from workloads import BlockManager

pa = pytest.importorskip("paged_kv_cache_350_amd")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(pa.LIB_PATH):
        pytest.fail("libpa.so is not built (python -m paged_kv_cache_350_amd.build)")


def test_block_manager_example():
    ex = load("block_manager_test.json")
    m = pa.NativeBlockManager(ex["total_pages"], ex["block_size"])
    pages = m.allocate(1, ex["num_tokens"])
    assert len(pages) == ex["pages_taken"]
    assert m.num_free() == ex["free_after_allocate"]
    m.free_sequence(1)
    assert m.num_free() == ex["free_after_free"]


def test_allocator_demo():
    ex = load("allocator_demo.json")
    m = pa.NativeBlockManager(ex["num_blocks"], ex["block_size"])
    pages = m.allocate(7, ex["num_tokens"])
    assert len(pages) == ex["pages_taken"]
    assert len(pages) * ex["block_size"] == ex["capacity_tokens"]


@pytest.mark.parametrize("name", ["page_table_figure.json", "flowchart_block_table.json"])
def test_block_table_figures(name):
    fig = load(name)
    bs, pages, n = fig["block_size"], fig["pages"], fig["num_tokens"]
    free = pages + [p for p in range(max(pages) + 1) if p not in pages]
    m = pa.NativeBlockManager(len(free), bs, free_order=free)
    assert m.allocate(3, n) == pages
    tables, lens = m.block_tables([3], len(pages) + 2, pad_page=99)
    assert tables[0].tolist() == pages + [99, 99] and lens.tolist() == [n]
    for t, page, off in fig["probes_token_page_offset"]:
        assert tables[0][t // bs] * bs + t % bs == page * bs + off


def test_page_table_figure_append_slot():
    """Growing the figure's 36-token prompt by one token writes page 2, offset 4."""
    fig = load("page_table_figure.json")
    free = fig["pages"] + [p for p in range(16) if p not in fig["pages"]]
    m = pa.NativeBlockManager(16, 16, free_order=free)
    m.allocate(0, fig["num_tokens"])
    slots, copies = m.append([0])
    assert slots.tolist() == [2 * 16 + 4] and len(copies) == 0


def test_exhaustion_is_an_error_and_changes_nothing():
    m = pa.NativeBlockManager(4, 16)
    with pytest.raises(MemoryError):
        m.allocate(1, 65)                              # 5 pages
    assert m.num_free() == 4 and m.num_seqs() == 0
    m.allocate(1, 48)                                  # 3 pages
    m.allocate(2, 16)                                  # 1 page: pool empty
    before = (m.free_list(), m.pages(1), m.pages(2), m.length(1), m.length(2))
    with pytest.raises(MemoryError):
        m.append([1, 2])                               # both open a block: 2 pages needed
    assert (m.free_list(), m.pages(1), m.pages(2), m.length(1), m.length(2)) == before
    with pytest.raises(KeyError):
        m.append([1, 5])                               # unknown id: nothing appended either
    assert m.length(1) == 48


def test_fifo_copy_on_write_and_refcounts():
    bs = 16
    m = pa.NativeBlockManager(10, bs)
    m.allocate(0, 20)                                   # pages 0, 1; page 1 holds 4 tokens
    m.fork(0, 1)
    m.fork(0, 2)
    assert [m.ref_count(p) for p in (0, 1)] == [3, 3]
    slots, copies = m.append([1, 2, 0])
    # 1 and 2 write into the shared page: copies to 2 and 3; 0 is then the last holder
    assert copies.tolist() == [[1, 2], [1, 3]]
    assert slots.tolist() == [2 * bs + 4, 3 * bs + 4, 1 * bs + 4]
    assert [m.ref_count(p) for p in range(4)] == [3, 1, 1, 1]
    m.free_sequence(0)
    assert m.free_list() == [4, 5, 6, 7, 8, 9, 1]      # freed page goes to the back
    with pytest.raises(ValueError):
        m.fork(1, 2)
    with pytest.raises(KeyError):
        m.fork(42, 43)


def test_same_sequence_twice_in_one_batch():
    bs = 4
    m = pa.NativeBlockManager(8, bs)
    m.allocate(0, 3)
    m.fork(0, 1)
    slots, copies = m.append([0, 0, 1])
    # token 3 of seq 0: shared page -> copy to page 1; token 4 opens page 2;
    # seq 1 then holds page 0 alone and writes in place
    assert copies.tolist() == [[0, 1]]
    assert slots.tolist() == [1 * bs + 3, 2 * bs + 0, 0 * bs + 3]
    assert m.pages(0) == [1, 2] and m.pages(1) == [0]


def _compare(py: BlockManager, nat, seqs):
    assert nat.free_list() == list(py.free)
    assert [nat.ref_count(p) for p in range(py.num_blocks)] == py.ref
    assert nat.num_seqs() == len(py.tables)
    for s in seqs:
        assert nat.pages(s) == py.tables[s]
        assert nat.length(s) == py.lengths[s]


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_the_host_manager(seed):
    rng = np.random.default_rng(100 + seed)
    num_blocks, bs = int(rng.integers(20, 200)), int(rng.choice([1, 4, 16, 32]))
    order = rng.permutation(num_blocks)
    py = BlockManager(num_blocks, bs, free_order=order)
    nat = pa.NativeBlockManager(num_blocks, bs, free_order=order)
    live, next_id = [], 0
    for _ in range(400):
        op = rng.choice(["alloc", "append", "fork", "free"], p=[0.25, 0.45, 0.15, 0.15])
        if op == "alloc":
            n = int(rng.integers(0, 5 * bs))
            try:
                py.allocate(next_id, n)
                ok = True
            except MemoryError:
                ok = False
            if ok:
                nat.allocate(next_id, n)
                live.append(next_id)
            else:
                with pytest.raises(MemoryError):
                    nat.allocate(next_id, n)
            next_id += 1
        elif op == "append" and live:
            batch = [int(x) for x in rng.choice(live, size=int(rng.integers(1, 6)))]
            state = (list(py.free), list(py.ref), {s: list(py.tables[s]) for s in live},
                     dict(py.lengths))
            try:
                want = [py.append_token(s) for s in batch]
                ok = True
            except MemoryError:
                ok = False
            if ok:
                slots, copies = nat.append(batch)
                assert slots.tolist() == want
                assert [tuple(c) for c in copies.tolist()] == py.take_copies()
            else:
                # the host manager fails part-way; the native one changes nothing --
                # roll the host manager back to compare the rest of the run
                with pytest.raises(MemoryError):
                    nat.append(batch)
                py.free = type(py.free)(state[0])
                py.ref = state[1]
                for s in live:
                    py.tables[s] = state[2][s]
                py.lengths = state[3]
                py.take_copies()
        elif op == "fork" and live:
            parent = int(rng.choice(live))
            py.fork(parent, next_id)
            nat.fork(parent, next_id)
            live.append(next_id)
            next_id += 1
        elif op == "free" and live:
            s = live.pop(int(rng.integers(0, len(live))))
            py.free_sequence(s)
            nat.free_sequence(s)
        _compare(py, nat, live)


@pytest.mark.parametrize("name", ["tiny", "llama3_8b", "llama3_70b", "prefix_share", "beam_fork",
                                  "long_context"])
def test_named_workloads_are_identical_under_the_native_manager(name):
    """Every table, slot, copy pair and poison mask of the full-size
    workloads comes out the same when the native manager assigns the pages."""
    a = workloads.by_name(name)
    b = workloads.by_name(name, manager=pa.NativeBlockManager)
    for field in ("context_lens", "block_tables", "append_slots", "append_seq", "copy_pairs",
                  "resident"):
        assert np.array_equal(getattr(a, field), getattr(b, field)), field
    assert a.pad_page == b.pad_page and a.num_blocks == b.num_blocks


def test_block_tables_feed_the_kernels_layout():
    m = pa.NativeBlockManager(64, 16)
    m.allocate(10, 40)
    m.allocate(11, 0)
    m.allocate(12, 17)
    t, lens = m.block_tables([12, 10, 11], 4, pad_page=63)
    assert lens.tolist() == [17, 40, 0]
    assert t.dtype == np.int32 and t.shape == (3, 4)
    assert t[0].tolist() == [3, 4, 63, 63] and t[1].tolist() == [0, 1, 2, 63] and t[2].tolist() == [63] * 4
    with pytest.raises(ValueError):
        m.block_tables([10], 2)
    with pytest.raises(KeyError):
        m.block_tables([99], 4)


def test_invalid_pools():
    with pytest.raises(ValueError):
        pa.NativeBlockManager(3, 16, free_order=[0, 0, 1])
    with pytest.raises(ValueError):
        pa.NativeBlockManager(0, 16)
    with pytest.raises(ValueError):
        pa.NativeBlockManager(8, 0)
    m = pa.NativeBlockManager(4, 16)
    m.allocate(1, 3)
    with pytest.raises(ValueError):
        m.allocate(1, 3)
    with pytest.raises(ValueError):
        m.allocate(2, -1)
    m.free_sequence(77)                                 # unknown: no-op


def test_in_place_table_updates_match_a_rebuild():
    """append() with tables keeps them equal to a fresh block_tables() call
    through block openings and copy-on-write, step after step."""
    rng = np.random.default_rng(7)
    bs, maxb = 16, 24
    m = pa.NativeBlockManager(600, bs, free_order=rng.permutation(600))
    m.allocate(0, 37)
    for child in range(1, 6):
        m.fork(0, child)                              # page 2 (5 tokens) shared by all six
    for s in range(6, 12):
        m.allocate(s, int(rng.integers(0, 90)))
    ids = np.arange(12, dtype=np.int64)
    tables, lens = m.block_tables(ids, maxb, pad_page=599)
    tables, lens = tables.copy(), lens.copy()
    total_copies = 0
    for step in range(150):
        order = rng.permutation(ids)
        rows = np.argsort(order)                      # row of each id in the permuted batch
        t_perm, l_perm = np.ascontiguousarray(tables[order]), lens[order].copy()
        slots, copies = m.append(order, t_perm, l_perm)
        total_copies += len(copies)
        tables, lens = t_perm[rows], l_perm[rows]
        want_t, want_l = m.block_tables(ids, maxb, pad_page=599)
        assert np.array_equal(tables, want_t) and np.array_equal(lens, want_l), step
        for i, s in enumerate(order):                  # ids are 0..11, so id s is row s
            pos = lens[s] - 1
            assert slots[i] == tables[s][pos // bs] * bs + pos % bs
    assert total_copies == 5                          # five of the six leave the shared page


def test_in_place_table_update_errors_change_nothing():
    m = pa.NativeBlockManager(40, 4)
    m.allocate(0, 7)
    m.allocate(1, 8)
    ids = np.array([0, 1], dtype=np.int64)
    t, l = m.block_tables(ids, 3)
    t, l = t.copy(), l.copy()
    with pytest.raises(ValueError):                   # duplicate ids with tables
        m.append(np.array([0, 0], dtype=np.int64), t, l)
    with pytest.raises(ValueError):                   # seq 1 would need a 4th page of 3
        for _ in range(5):
            m.append(ids, t, l)
    assert m.length(0) == 7 + 4 and m.length(1) == 8 + 4   # the failing call changed nothing
    assert np.array_equal(t, m.block_tables(ids, 3)[0])


def test_shared_prefix_of_forks_and_beams():
    """The tokens a set of sequences holds in the same pages: all of a forked
    prompt's whole pages; copy-on-write of the shared tail page ends the
    sharing there; unrelated sequences share nothing."""
    m = pa.NativeBlockManager(64, 16)
    m.allocate(0, 100)                        # 7 pages, the last holding 4 tokens
    for c in (1, 2, 3):
        m.fork(0, c)
    assert m.shared_prefix([1, 2, 3]) == 96   # whole pages, capped by the 100 tokens
    assert m.shared_prefix([2]) == 96
    m.append_token(1)                         # copy-on-write of page 6 for sequence 1
    assert m.shared_prefix([1, 2, 3]) == 96
    for _ in range(60):
        m.append_token(2)
        m.append_token(3)
    assert m.shared_prefix([2, 3]) == 96      # both copied page 6 (CoW), then own pages
    m.allocate(9, 40)
    assert m.shared_prefix([9, 1]) == 0
    assert m.shared_prefix([]) == 0
    with pytest.raises(KeyError):
        m.shared_prefix([1, 77])
    m.close()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_shared_prefix_agrees_with_the_tables(seed):
    """The manager's answer equals the one read off its own block tables
    (leading entries equal in every row, whole pages, capped by the shortest
    context)."""
    rng = np.random.default_rng(seed)
    bs = 16
    m = pa.NativeBlockManager(4096, bs)
    m.allocate(0, int(rng.integers(1, 900)))
    ids = list(range(1, 9))
    for c in ids:
        m.fork(0, c)
    for _ in range(200):
        m.append_token(int(rng.choice(ids)))
    for k in range(1, len(ids) + 1):
        pick = [int(x) for x in rng.choice(ids, size=k, replace=False)]
        tables, lens = m.block_tables(pick, 128, pad_page=4095)
        assert m.shared_prefix(pick) == pa.shared_prefix_len(tables, lens, bs), pick
    m.close()


def test_prefix_groups_of_a_batch():
    """Two forked prompts, a loner between them, then a single fork: each
    maximal run starting on one page and sharing a whole page is a group;
    the sequences between two such runs share nothing, one group for the
    lot; the bounds cover only the groups that share."""
    m = pa.NativeBlockManager(256, 16)
    m.allocate(100, 200)                     # prompt A: 12 full pages + 8 tokens
    m.allocate(200, 64)                      # prompt B: 4 full pages
    for c in (1, 2, 3):
        m.fork(100, c)
    for c in (5, 6):
        m.fork(200, c)
    m.allocate(4, 30)                        # on its own
    m.allocate(8, 17)                        # on its own
    m.fork(200, 7)
    for s in (1, 2, 3, 5, 6, 7):
        m.append_token(s)                    # copy-on-write of A's tail page; B's is full
    batch = [1, 2, 3, 4, 5, 6, 7]
    gs, gl, sl, max_group, max_shared = m.prefix_groups(batch)
    assert gs.tolist() == [0, 3, 4, 7]
    assert gl.tolist() == [192, 0, 64]
    assert sl.tolist() == [192, 192, 192, 0, 64, 64, 64]
    assert (max_group, max_shared) == (3, 192)
    for (a, e), S in zip(zip(gs[:-1], gs[1:]), gl):
        if e - a >= 2:
            assert S == m.shared_prefix(batch[a:e])
    # two loners together, and a lone member of a forked prompt: one group sharing nothing
    gs, gl, sl, max_group, max_shared = m.prefix_groups([4, 8, 1, 5, 6, 7])
    assert gs.tolist() == [0, 3, 6] and gl.tolist() == [0, 64] and sl.tolist() == [0, 0, 0, 64, 64, 64]
    assert (max_group, max_shared) == (3, 64)
    assert [x.tolist() if hasattr(x, "tolist") else x for x in m.prefix_groups([4])] == [[0, 1], [0], [0], 1, 0]
    assert [x.tolist() if hasattr(x, "tolist") else x for x in m.prefix_groups([])] == [[0], [], [], 1, 0]
    with pytest.raises(KeyError):
        m.prefix_groups([1, 99])
    m.close()
