"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and
check that at least one pin catches each of them."""

import math

import numpy as np
import pytest

import oracle
import oracle.paged_attention as pa
from oracle.formats import to_f64
from oracle_pins import ALL_PINS


def _attend_no_scale(qvec, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = K @ qvec
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def _attend_wrong_sign(qvec, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = scale * (K @ qvec)
    p = np.exp(s.min() - s)
    return (p @ V) / p.sum()


def _attend_no_normalise(qvec, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = scale * (K @ qvec)
    p = np.exp(s - s.max())
    return p @ V


def _attend_sqrt_scale_again(qvec, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = scale * (K @ qvec) / math.sqrt(K.shape[1])
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def _gather_factory(kind):
    def gather(k_cache, v_cache, table_row, context_len, block_size, dtype):
        L = int(context_len)
        nb, hkv, nchunk, bs, x = k_cache.shape
        d = nchunk * x
        pos = np.arange(L)
        offs = pos % bs
        blocks = pos // bs
        if kind == "offset_off_by_one":
            offs = (pos + 1) % bs
        if kind == "block_index_uses_offset":
            blocks = pos % max(1, -(-L // bs))
        pages = np.asarray(table_row, dtype=np.int64)[blocks] if L else np.zeros(0, np.int64)
        if kind == "identity_pages":
            pages = blocks
        k = k_cache[pages, :, :, offs, :]
        if kind == "chunk_axes_swapped":
            k = np.swapaxes(k, 2, 3)
        v = v_cache[pages, :, :, offs]
        K = to_f64(np.ascontiguousarray(k), dtype).reshape(L, hkv, d)
        V = to_f64(np.ascontiguousarray(v), dtype).reshape(L, hkv, d)
        if kind == "k_and_v_swapped":
            K, V = V, K
        return K, V
    return gather


def _attend_default_scale(qvec, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = (K @ qvec) / math.sqrt(K.shape[1])           # the given scale ignored
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


_real_gather = pa.gather_sequence


def _gather_drops_newest(k_cache, v_cache, table_row, context_len, block_size, dtype):
    return _real_gather(k_cache, v_cache, table_row, max(int(context_len) - 1, 0), block_size, dtype)


_real_decode = pa.decode


def _decode_wrong_row(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype, seqs=None):
    tables = np.roll(np.asarray(block_tables), 1, axis=0)        # sequence b reads b - 1's table
    return _real_decode(q, k_cache, v_cache, tables, context_lens, scale, block_size, dtype, seqs)


MUTANTS = {
    "given_scale_ignored": ("attend", _attend_default_scale),
    "newest_token_dropped": ("gather_sequence", _gather_drops_newest),
    "neighbouring_table_row": ("decode", _decode_wrong_row),
    "scale_dropped": ("attend", _attend_no_scale),
    "softmax_sign": ("attend", _attend_wrong_sign),
    "no_normalisation": ("attend", _attend_no_normalise),
    "scale_applied_twice": ("attend", _attend_sqrt_scale_again),
    "gqa_modulo_mapping": ("kv_head_of", lambda h, g: h % g),
    "gqa_first_head_only": ("kv_head_of", lambda h, g: 0),
    "offset_off_by_one": ("gather_sequence", _gather_factory("offset_off_by_one")),
    "block_index_uses_offset": ("gather_sequence", _gather_factory("block_index_uses_offset")),
    "identity_pages": ("gather_sequence", _gather_factory("identity_pages")),
    "chunk_axes_swapped": ("gather_sequence", _gather_factory("chunk_axes_swapped")),
    "k_and_v_swapped": ("gather_sequence", _gather_factory("k_and_v_swapped")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(pa, attr, fn)
    if hasattr(oracle, attr):                 # the pins call the package-level name
        monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(oracle)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin in ALL_PINS:
        pin(oracle)
