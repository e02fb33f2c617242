"""Append scatter and page copy oracles pinned to explicit element loops, the
page-table figure and bit preservation (CPU only)."""

import json
import os

import numpy as np

import oracle
from oracle_pins import contiguous_to_paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_append_matches_elementwise_writes_and_keeps_bits():
    rng = np.random.default_rng(1)
    nb, hkv, d, bs, x = 5, 2, 16, 16, 4
    kc = rng.standard_normal((nb, hkv, d // x, bs, x)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, d, bs)).astype(np.float32)
    kc[3, :, :, 7, :] = np.float32(np.nan)       # a NaN payload elsewhere must survive
    kn = rng.standard_normal((4, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((4, hkv, d)).astype(np.float32)
    # the padding slot -1 would wrap to the pool's very last slot: keep that
    # slot unwritten, so a write through a negative slot shows
    slots = np.array([2 * bs + 5, -1, 0, nb * bs - 2], np.int64)
    k2, v2 = oracle.kv_append(kn, vn, slots, kc, vc, bs)
    want_k, want_v = kc.copy(), vc.copy()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        page, off = int(s) // bs, int(s) % bs
        for h in range(hkv):
            for e in range(d):
                want_k[page, h, e // x, off, e % x] = kn[i, h, e]
                want_v[page, h, e, off] = vn[i, h, e]
    assert np.array_equal(k2.view(np.uint32), want_k.view(np.uint32))
    assert np.array_equal(v2.view(np.uint32), want_v.view(np.uint32))
    # the inputs are not modified
    assert np.isnan(kc[3, 0, 0, 7, 0]) and not np.array_equal(k2, kc)


def test_append_then_gather_returns_the_row_at_its_position():
    """Slot = page * bs + offset with the page from the figure's table."""
    fig = json.load(open(os.path.join(GOLDEN, "page_table_figure.json")))
    bs, pages = fig["block_size"], fig["pages"]
    nb, hkv, d, x = 16, 1, 8, 4
    kc = np.full((nb, hkv, d // x, bs, x), np.nan, np.float32)
    vc = np.full((nb, hkv, d, bs), np.nan, np.float32)
    rng = np.random.default_rng(2)
    rows_k = rng.standard_normal((fig["num_tokens"], hkv, d)).astype(np.float32)
    rows_v = rng.standard_normal((fig["num_tokens"], hkv, d)).astype(np.float32)
    for t, page, off in fig["probes_token_page_offset"]:
        assert oracle.resolve_slot(pages, t, bs) == (page, off)
    slots = np.array([pages[t // bs] * bs + t % bs for t in range(fig["num_tokens"])], np.int64)
    kc, vc = oracle.kv_append(rows_k, rows_v, slots, kc, vc, bs)
    K, V = oracle.gather_sequence(kc, vc, pages, fig["num_tokens"], bs, "f32")
    assert np.array_equal(K, rows_k.astype(np.float64))
    assert np.array_equal(V, rows_v.astype(np.float64))
    # the figure's last block holds 4 tokens: the rest of page 2 stays unwritten
    assert np.isnan(vc[2, :, :, fig["last_block_fill"]:]).all()


def test_bf16_append_is_a_bit_copy():
    rng = np.random.default_rng(3)
    nb, hkv, d, bs = 3, 2, 16, 32
    kc = rng.integers(0, 2 ** 16, (nb, hkv, d // 8, bs, 8), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, (nb, hkv, d, bs), dtype=np.uint16)
    kn = rng.integers(0, 2 ** 16, (2, hkv, d), dtype=np.uint16)
    vn = rng.integers(0, 2 ** 16, (2, hkv, d), dtype=np.uint16)
    k2, v2 = oracle.kv_append(kn, vn, np.array([33, 95], np.int64), kc, vc, bs)
    assert np.array_equal(k2[1, :, :, 1, :].reshape(hkv, d), kn[0])
    assert np.array_equal(v2[2, :, :, 31], vn[1])
    mask = np.ones(k2.shape, bool)
    mask[1, :, :, 1, :] = False
    mask[2, :, :, 31, :] = False
    assert np.array_equal(k2[mask], kc[mask])


def test_copy_blocks_is_simultaneous_and_exact():
    rng = np.random.default_rng(4)
    nb, hkv, d, bs, x = 6, 2, 8, 16, 4
    kc = rng.standard_normal((nb, hkv, d // x, bs, x)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, d, bs)).astype(np.float32)
    vc[1, 0, 0, 3] = np.float32(np.nan)
    pairs = np.array([[1, 4], [0, 5], [1, 2]], np.int64)     # one source, two copies
    k2, v2 = oracle.copy_blocks(kc, vc, pairs)
    for s, t in pairs:
        assert np.array_equal(k2[t].view(np.uint32), kc[s].view(np.uint32))
        assert np.array_equal(v2[t].view(np.uint32), vc[s].view(np.uint32))
    for p in (0, 1, 3):
        assert np.array_equal(k2[p].view(np.uint32), kc[p].view(np.uint32))
    # pairs read the pre-call contents: a chain a->b, b->c copies the old b
    k3, _ = oracle.copy_blocks(kc, vc, np.array([[0, 1], [1, 2]], np.int64))
    assert np.array_equal(k3[2], kc[1]) and np.array_equal(k3[1], kc[0])


def test_paged_scatter_helper_matches_gather():
    """The test-side scatter and the oracle's gather are inverse of each other."""
    rng = np.random.default_rng(5)
    K = rng.standard_normal((50, 2, 8)).astype(np.float32)
    V = rng.standard_normal((50, 2, 8)).astype(np.float32)
    table = [3, 0, 6, 1]
    kc, vc = contiguous_to_paged(K, V, table, 16, 8, 4)
    K2, V2 = oracle.gather_sequence(kc, vc, table, 50, 16, "f32")
    assert np.array_equal(K2, K.astype(np.float64)) and np.array_equal(V2, V.astype(np.float64))
