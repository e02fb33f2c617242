"""The synthetic workloads have the stated shapes, statistics and structure."""

import math

import numpy as np
import pytest
import torch

import workloads as W


def _check_structure(w):
    bs = w.block_size
    assert w.block_tables.dtype == np.int32 and w.context_lens.dtype == np.int32
    for b in range(w.num_seqs):
        L = int(w.context_lens[b])
        n = -(-L // bs)
        row = w.block_tables[b]
        assert (row[:n] >= 0).all() and (row[:n] < w.num_blocks).all()
        assert (row[n:] == w.pad_page).all()
    assert not w.resident[w.pad_page].any()
    # appended slots are free before the step (or become private by copy first)
    dst = set(w.copy_pairs[:, 1].tolist())
    for s in w.append_slots:
        page, off = divmod(int(s), bs)
        assert not w.resident[page, off] or page in dst
    assert len(set(w.append_slots.tolist())) == len(w.append_slots)
    src, dsts = set(w.copy_pairs[:, 0].tolist()), w.copy_pairs[:, 1].tolist()
    assert len(set(dsts)) == len(dsts) and not (src & set(dsts))


def test_tiny():
    w = W.tiny()
    assert w.context_lens.tolist() == [36, 42] and w.num_blocks == 16
    assert (w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.dtype) == (4, 4, 64, 16, "f32")
    assert w.scale == 0.125
    _check_structure(w)
    # 6 pages used, 10 spare
    used = set(w.block_tables[0, :3].tolist()) | set(w.block_tables[1, :3].tolist())
    assert len(used) == 6 and w.resident.sum() == 35 + 41
    assert w.algorithmic_kv_bytes() == 78 * 2 * 4 * 64 * 4 == 159744


def test_llama3_8b():
    w = W.llama3_8b()
    assert w.num_seqs == 64 and (w.num_heads, w.num_kv_heads, w.head_dim) == (32, 8, 128)
    L = w.context_lens
    assert L.min() >= 512 and L.max() <= 4096
    need = sum(-(-int(x) // 16) for x in L)
    assert w.num_blocks == math.ceil(1.1 * need)
    assert w.kv_bytes_per_token() == 4096
    _check_structure(w)
    assert W.llama3_8b().context_lens.tolist() == L.tolist()       # seeded


def test_llama3_70b():
    w = W.llama3_70b()
    L = w.context_lens
    assert w.num_seqs == 256 and (w.num_heads, w.num_kv_heads) == (64, 8)
    assert L.min() >= 64 and L.max() <= 8192
    assert 1100 < np.median(L) < 2000
    _check_structure(w)


def test_long_context():
    w = W.long_context()
    assert w.context_lens.tolist() == [32768] * 8 and w.num_blocks == 18023
    assert w.partition_size == 512
    assert w.algorithmic_kv_bytes() == 1 << 30
    _check_structure(w)


def test_prefix_share():
    w = W.prefix_share()
    assert w.num_seqs == 100 and w.block_size == 32
    suffix = w.context_lens - 10000
    assert suffix.min() >= 0 and suffix.max() <= 512
    shared = w.extra["shared_pages"]
    assert len(shared) == 313
    # every sequence starts with the 312 full shared pages
    assert (w.block_tables[:, :312] == np.array(shared[:312])).all()
    # writers into the partly filled shared page copy it first, except its last holder
    assert all(src == shared[312] for src in w.copy_pairs[:, 0])
    writers = int((suffix > 0).sum())
    assert len(w.copy_pairs) in (writers, writers - 1)
    assert len(w.append_slots) == int(suffix.sum())
    _check_structure(w)
    assert w.unique_kv_bytes() < w.algorithmic_kv_bytes() / 10


def test_beam_fork():
    w = W.beam_fork()
    assert w.num_seqs == 8 and (w.context_lens == 32774).all()
    assert len(w.copy_pairs) == 7
    assert (w.block_tables[:, :1024] == w.block_tables[0, :1024]).all()
    _check_structure(w)


def test_copy_probe_pairs():
    pairs = W.copy_probe()
    assert pairs.shape == (7 * 1024, 2)
    assert len(set(pairs[:, 1].tolist())) == len(pairs)
    assert not (set(pairs[:, 0].tolist()) & set(pairs[:, 1].tolist()))


def test_make_tensors_poisons_non_resident_slots():
    w = W.tiny()
    t = W.make_tensors(w, "cpu")
    kc, vc = t["k_cache"], t["v_cache"]
    assert kc.shape == w.k_cache_shape() and vc.shape == w.v_cache_shape()
    res = torch.from_numpy(w.resident)
    nan_k = torch.isnan(kc).all(dim=4).all(dim=2).all(dim=1)          # [nb, bs]
    fin_k = torch.isfinite(kc).all(dim=4).all(dim=2).all(dim=1)
    assert torch.equal(fin_k, res) and torch.equal(nan_k, ~res)
    nan_v = torch.isnan(vc).all(dim=2).all(dim=1)
    assert torch.equal(nan_v, ~res)
    assert t["q"].dtype == torch.float32 and t["q"].shape == (2, 4, 64)
    # same seed, same values
    t2 = W.make_tensors(w, "cpu")
    assert torch.equal(t["q"], t2["q"])


def test_prompt_chunk_and_multi_flops():
    """The chunked-prefill workload's shape, and the multi-query flop count
    against positions counted one by one: query j of a sequence with n new
    tokens sees L - n + j + 1 positions, each costing 4 D flops per head."""
    w = W.prompt_chunk()
    assert (w.num_seqs, w.max_query_len, w.max_context_len) == (8, 512, 4096)
    assert (w.num_heads, w.num_kv_heads, w.head_dim, w.block_size) == (32, 8, 128, 16)
    assert len(w.append_slots) == 8 * 512
    small = W.multi_custom("flops", 1, [5, 3, 7], [2, 3, 0], 8, 2, 64, 16)
    seen = 0
    for L, n in ((5, 2), (3, 3), (7, 0)):
        for j in range(n):
            seen += L - n + j + 1
    assert seen == (4 + 5) + (1 + 2 + 3)
    assert small.multi_flops() == 4 * 64 * 8 * seen
    assert w.multi_flops() == 4 * 128 * 32 * 8 * sum(3584 + j + 1 for j in range(512))
