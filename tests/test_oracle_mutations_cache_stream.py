"""Planted mistakes in the append, page-copy and streaming oracles (on the
CPU, via monkeypatch): each must fail at least one of the pins in
test_oracle_cache_ops.py / test_oracle_streaming.py, run here as plain
functions."""

import numpy as np
import pytest

import oracle
import oracle.streaming as st
import test_oracle_cache_ops as cache_pins
import test_oracle_streaming as stream_pins
from oracle.cache_ops import _bits


def _append_factory(kind):
    def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, block_size):
        kc, vc = _bits(k_cache).copy(), _bits(v_cache).copy()
        kn, vn = _bits(k_new), _bits(v_new)
        nb, hkv, nchunk, bs, x = kc.shape
        if kind == "k_and_v_swapped":
            kn, vn = vn, kn
        for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
            if slot < 0 and kind != "negative_slot_written":
                continue
            page, off = divmod(int(slot), bs)
            if kind == "page_and_offset_swapped":
                page, off = off % nb, page % bs
            row = kn[i].reshape(hkv, nchunk, x)
            if kind == "chunk_layout_transposed":
                row = kn[i].reshape(hkv, x, nchunk).swapaxes(1, 2)
            kc[page, :, :, off, :] = row
            vc[page, :, :, off] = vn[i]
        if np.asarray(k_cache).dtype == np.float32:
            return kc.view(np.float32), vc.view(np.float32)
        return kc, vc
    return kv_append


def _copy_factory(kind):
    def copy_blocks(k_cache, v_cache, pairs):
        kb, vb = _bits(k_cache), _bits(v_cache)
        kc, vc = kb.copy(), vb.copy()
        for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
            if kind == "source_and_destination_swapped":
                src, dst = dst, src
            if kind == "copies_in_sequence":
                kc[dst], vc[dst] = kc[src], vc[src]        # reads pages already overwritten
            else:
                kc[dst] = kb[src]
                if kind != "v_not_copied":
                    vc[dst] = vb[src]
        if np.asarray(k_cache).dtype == np.float32:
            return kc.view(np.float32), vc.view(np.float32)
        return kc, vc
    return copy_blocks


def _online_no_rescale(qvec, K, V, scale, chunk):
    m, l = -np.inf, 0.0
    acc = np.zeros(V.shape[1], dtype=np.float64)
    for start in range(0, K.shape[0], chunk):
        s = scale * (K[start:start + chunk] @ qvec)
        m_new = max(m, float(s.max()))
        alpha = np.exp(m - m_new)
        p = np.exp(s - m_new)
        l = l * alpha + float(p.sum())
        acc = acc + p @ V[start:start + chunk]              # accumulator left at the old reference
        m = m_new
    return m, l, acc


def _split_unweighted(qb, K, V, scale, group, partition, chunk):
    hq, d = qb.shape
    out = np.zeros((hq, d), dtype=np.float64)
    if K.shape[0] == 0:
        return out
    for h in range(hq):
        g = h // group
        parts = [st._online(qb[h], K[s:s + partition, g, :], V[s:s + partition, g, :], scale, chunk)
                 for s in range(0, K.shape[0], partition)]
        out[h] = sum(p[2] for p in parts) / sum(p[1] for p in parts)   # partitions' maxima ignored
    return out


CACHE_PINS = [
    cache_pins.test_append_matches_elementwise_writes_and_keeps_bits,
    cache_pins.test_append_then_gather_returns_the_row_at_its_position,
    cache_pins.test_bf16_append_is_a_bit_copy,
    cache_pins.test_copy_blocks_is_simultaneous_and_exact,
]

STREAM_PINS = [
    lambda: stream_pins.test_online_equals_plain(517, 32),
    lambda: stream_pins.test_online_equals_plain(2049, 64),
    lambda: stream_pins.test_split_merge_equals_plain(5000, 512),
    lambda: stream_pins.test_split_merge_equals_plain(3000, 256),
    stream_pins.test_split_with_wildly_different_partition_maxima,
]

MUTANTS = {
    "append_page_and_offset_swapped": (oracle, "kv_append", _append_factory("page_and_offset_swapped"), CACHE_PINS),
    "append_k_and_v_swapped": (oracle, "kv_append", _append_factory("k_and_v_swapped"), CACHE_PINS),
    "append_chunk_layout_transposed": (oracle, "kv_append", _append_factory("chunk_layout_transposed"), CACHE_PINS),
    "append_negative_slot_written": (oracle, "kv_append", _append_factory("negative_slot_written"), CACHE_PINS),
    "copy_in_sequence": (oracle, "copy_blocks", _copy_factory("copies_in_sequence"), CACHE_PINS),
    "copy_direction_swapped": (oracle, "copy_blocks", _copy_factory("source_and_destination_swapped"), CACHE_PINS),
    "copy_v_not_copied": (oracle, "copy_blocks", _copy_factory("v_not_copied"), CACHE_PINS),
    "online_no_accumulator_rescale": (st, "_online", _online_no_rescale, STREAM_PINS),
    "merge_ignores_partition_maxima": (oracle, "split_decode_sequence", _split_unweighted, STREAM_PINS),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    module, attr, fn, pins = MUTANTS[name]
    monkeypatch.setattr(module, attr, fn)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught, f"no pin caught the planted mistake {name}"


def test_pins_pass_on_the_oracle_as_it_is():
    for pin in CACHE_PINS + STREAM_PINS:
        pin()
