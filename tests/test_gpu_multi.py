"""pa_decode_multi (several new tokens per sequence, causal among them) on
the GPU, through the C ABI.

Every case appends the new tokens' K/V rows with pa_kv_append and then runs
pa_decode_multi.  The oracle takes the caches as generated (before the
append), applies its own append of the same rows and computes
oracle.decode_multi in float64, so no oracle input comes from the device.
Tolerances are the decode ones (bf16: max-abs 2e-2, relative L2 5e-3).

Two kernels serve the call: below 64 query columns per (sequence, kv head)
(G heads x n new tokens) the per-wave-loads multi-query kernel, from 64 on
(a prompt chunk) the LDS-staged kernel with causal rows.  Each has tests of
its own below; the shared ones cover whichever the shape picks."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bits_equal, check_close, out_f64, require_gpu, say, storage_np

pytestmark = pytest.mark.gpu

# context lengths (new tokens included) around chunk and partition edges, and
# the new tokens of each: 0, 1, all of the context, and more than fill a tile
LENS = [1, 5, 16, 17, 31, 32, 33, 64, 100, 257, 513, 700]
NEWS = [1, 5, 3, 0, 8, 1, 16, 7, 2, 12, 5, 9]

SHAPES = [  # (block_size, num_heads, num_kv_heads, head_dim)
    (16, 32, 8, 128),
    (32, 32, 8, 128),
    (16, 64, 8, 128),
    (32, 8, 2, 64),
    (16, 16, 16, 128),
    (16, 16, 1, 64),
]
PARTS = [-1, 0, 64, 256]


def run_gpu(pa, w, t, partition_size=0, reuse="auto"):
    pa.kv_append(t["k_new"], t["v_new"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    return pa.decode_multi(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                           t["query_start"], w.scale, w.max_context_len, w.max_query_len,
                           partition_size=partition_size, reuse=reuse)


def oracle_multi(w, kc0, vc0, q, seqs=None):
    """Oracle append of the step's rows into the generated caches, then the
    multi-query oracle (rows of sequences outside ``seqs`` stay zero)."""
    keep = np.ones(len(w.append_seq), dtype=bool) if seqs is None else np.isin(w.append_seq, list(seqs))
    kc, vc = oracle.kv_append(w._k_new[keep], w._v_new[keep], w.append_slots[keep], kc0, vc0, w.block_size)
    return oracle.decode_multi(q, kc, vc, w.block_tables, w.context_lens, w.query_start, w.scale,
                               w.block_size, "bf16", seqs=seqs)


def prepare(w):
    t = W.make_tensors(w, "cuda")
    w._k_new, w._v_new = storage_np(t["k_new"]), storage_np(t["v_new"])
    return t, storage_np(t["k_cache"]), storage_np(t["v_cache"]), storage_np(t["q"])


def narrow_news(group):
    """NEWS capped so that group x n stays below 64 columns: the per-wave
    kernel, whatever the head shape."""
    return [min(n, max(1, 63 // group)) for n in NEWS]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_multi_narrow_matches_oracle(shape):
    pa = require_gpu()
    bs, hq, hkv, d = shape
    news = narrow_news(hq // hkv)
    assert (hq // hkv) * max(news) < 64
    w = W.multi_custom("narrow_multi", 47, LENS, news, hq, hkv, d, bs)
    t, kc0, vc0, q = prepare(w)
    ref = oracle_multi(w, kc0, vc0, q)
    for P in PARTS:
        t2 = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        say("narrow multi", shape, "partition", P, w.summary())
        out = run_gpu(pa, w, t2, partition_size=P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"narrow {shape} P={P}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_multi_matches_oracle(shape):
    pa = require_gpu()
    bs, hq, hkv, d = shape
    w = W.multi_custom("ragged_multi", 41, LENS, NEWS, hq, hkv, d, bs)
    t, kc0, vc0, q = prepare(w)
    ref = oracle_multi(w, kc0, vc0, q)
    for P in PARTS:
        t2 = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        say("multi", shape, "partition", P, w.summary())
        out = run_gpu(pa, w, t2, partition_size=P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"{shape} P={P}")


def test_one_new_token_is_bit_identical_to_decode():
    """With n = 1 everywhere the multi-query kernel does the decode kernel's
    arithmetic in the same order: given the same partition size (the two
    entry points' defaults differ), outputs agree bit for bit with
    pa_decode's streaming path, single pass and split."""
    pa = require_gpu()
    lens = [1, 17, 33, 300, 513, 1024, 2000, 4095]
    w = W.multi_custom("one_new", 42, lens, [1] * len(lens), 32, 8, 128, 16)
    for P in (-1, 256, 1024):
        t, _, _, _ = prepare(w)
        say("n=1 vs decode, partition", P)
        pa.kv_append(t["k_new"], t["v_new"], t["slot_mapping"], t["k_cache"], t["v_cache"])
        a = pa.decode_multi(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                            t["query_start"], w.scale, w.max_context_len, 1, partition_size=P)
        b = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"], w.scale,
                      w.max_context_len, partition_size=P, kernel="mfma", reuse="stream")
        torch.cuda.synchronize()
        assert bits_equal(a, b), P


def test_wide_queries_span_column_groups():
    """16 query heads per kv head x 8 new tokens = 128 columns: four column
    groups of two tiles, each reading the pages on its own."""
    pa = require_gpu()
    w = W.multi_custom("wide", 43, [8, 40, 129, 600], [8, 8, 3, 8], 64, 4, 128, 16)
    t, kc0, vc0, q = prepare(w)
    ref = oracle_multi(w, kc0, vc0, q)
    for P in (-1, 64):
        t2 = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        say("wide, partition", P)
        out = run_gpu(pa, w, t2, partition_size=P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"wide P={P}")


def test_shared_and_stream_paths_agree():
    pa = require_gpu()
    w = W.multi_custom("paths", 44, LENS, NEWS, 32, 8, 128, 16)
    outs = []
    for reuse in ("stream", "shared"):
        t, _, _, _ = prepare(w)
        say("reuse", reuse)
        outs.append(run_gpu(pa, w, t, partition_size=64, reuse=reuse))
    torch.cuda.synchronize()
    assert bits_equal(outs[0], outs[1])


def test_rows_outside_the_sequences_are_untouched_in_one_pass():
    """Query rows past query_start[num_seqs] are not written (single pass)."""
    pa = require_gpu()
    w = W.multi_custom("tail_rows", 45, [40, 70], [3, 2], 32, 8, 128, 16)
    t, kc0, vc0, q = prepare(w)
    pa.kv_append(t["k_new"], t["v_new"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    q_big = torch.cat([t["q"], t["q"][:2]]).contiguous()
    out = torch.full_like(q_big, 7.0)
    pa.decode_multi(q_big, t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"], t["query_start"],
                    w.scale, w.max_context_len, w.max_query_len, out=out, partition_size=-1)
    torch.cuda.synchronize()
    ref = oracle_multi(w, kc0, vc0, q)
    check_close(out_f64(out[:5]), ref, "bf16", "covered rows")
    assert bool((out[5:] == 7.0).all())


def test_spec_verify_full_size_sampled():
    """The speculative-verification batch at full size (64 sequences, 5
    queries each, contexts up to 4,096) in the benchmark's launch
    configuration; 12 sampled sequences checked against the oracle."""
    pa = require_gpu()
    w = W.spec_verify()
    t, kc0, vc0, q = prepare(w)
    say("spec_verify full size", w.summary())
    out = run_gpu(pa, w, t)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    seqs = sorted(rng.choice(w.num_seqs, size=12, replace=False).tolist())
    ref = oracle_multi(w, kc0, vc0, q, seqs=seqs)
    rows = np.concatenate([np.arange(w.query_start[b], w.query_start[b + 1]) for b in seqs])
    check_close(out_f64(out)[rows], ref[rows], "bf16", "spec_verify sampled")


@pytest.mark.parametrize("shape", [(16, 32, 8, 128), (32, 8, 2, 64), (16, 16, 1, 64)],
                         ids=lambda s: "-".join(map(str, s)))
def test_fused_append_equals_append_then_multi(shape):
    """pa_decode_multi_append = pa_kv_append + pa_decode_multi, bit for bit
    (outputs and whole caches, NaN poison included), and within tolerance of
    the oracle; new tokens straddle pages, partitions and column groups."""
    pa = require_gpu()
    bs, hq, hkv, d = shape
    w = W.multi_custom("fused_multi", 46, LENS, NEWS, hq, hkv, d, bs)
    t, kc0, vc0, q = prepare(w)
    ref = oracle_multi(w, kc0, vc0, q)
    for P in (-1, 0, 64):
        a = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        b = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        say("fused multi append", shape, "partition", P)
        out_a = run_gpu(pa, w, a, partition_size=P)
        out_b = pa.decode_multi(b["q"], b["k_cache"], b["v_cache"], b["block_tables"], b["context_lens"],
                                b["query_start"], w.scale, w.max_context_len, w.max_query_len, partition_size=P,
                                k_new=b["k_new"], v_new=b["v_new"])
        torch.cuda.synchronize()
        assert bits_equal(out_a, out_b), P
        assert bits_equal(a["k_cache"], b["k_cache"]) and bits_equal(a["v_cache"], b["v_cache"]), P
        check_close(out_f64(out_b), ref, "bf16", f"fused {shape} P={P}")


def test_fused_append_many_new_rows():
    """The per-wave kernel (one head per kv head, so 40 new tokens stay
    below 64 columns) with more new rows per workgroup than one wave's LDS
    slice holds (17 to 32: the workgroup copies them to LDS before its loop)
    and more than that (stored first): bit-identical to pa_kv_append +
    pa_decode_multi and within tolerance of the oracle."""
    pa = require_gpu()
    w = W.multi_custom("many_new", 50, [20, 45, 300, 700, 33], [20, 33, 17, 40, 32], 8, 8, 128, 16)
    t, kc0, vc0, q = prepare(w)
    ref = oracle_multi(w, kc0, vc0, q)
    for P in (-1, 64):
        a = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        b = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        say("fused multi append, many new rows, partition", P)
        out_a = run_gpu(pa, w, a, partition_size=P)
        out_b = pa.decode_multi(b["q"], b["k_cache"], b["v_cache"], b["block_tables"], b["context_lens"],
                                b["query_start"], w.scale, w.max_context_len, w.max_query_len, partition_size=P,
                                k_new=b["k_new"], v_new=b["v_new"])
        torch.cuda.synchronize()
        assert bits_equal(out_a, out_b), P
        assert bits_equal(a["k_cache"], b["k_cache"]) and bits_equal(a["v_cache"], b["v_cache"]), P
        check_close(out_f64(out_b), ref, "bf16", f"many new rows P={P}")


def test_fused_append_skips_pages_outside_the_pool():
    """A block-table entry outside the pool at a new token's position: that
    row is not written anywhere (as pa_kv_append skips an out-of-range slot);
    every other new row lands where the oracle puts it."""
    pa = require_gpu()
    w = W.multi_custom("bad_page", 47, [40, 70, 20], [5, 3, 4], 32, 8, 128, 16)
    t, kc0, vc0, q = prepare(w)
    bad_seq, bad_pos = 1, 69                       # the last new token of sequence 1
    tables = w.block_tables.copy()
    tables[bad_seq, bad_pos // 16] = w.num_blocks + 3
    bt = torch.from_numpy(tables).cuda()
    say("fused multi append, page outside the pool")
    pa.decode_multi(t["q"], t["k_cache"], t["v_cache"], bt, t["context_lens"], t["query_start"], w.scale,
                    w.max_context_len, w.max_query_len, partition_size=-1, k_new=t["k_new"], v_new=t["v_new"])
    torch.cuda.synchronize()
    slots = w.append_slots.copy()
    page_of_bad = w.block_tables[bad_seq, bad_pos // 16]
    keep = (slots // 16) != page_of_bad           # every row of the page the bad entry stood for
    kc, vc = oracle.kv_append(w._k_new[keep], w._v_new[keep], slots[keep], kc0, vc0, 16)
    assert np.array_equal(storage_np(t["k_cache"]).view(np.uint16), kc.view(np.uint16))
    assert np.array_equal(storage_np(t["v_cache"]).view(np.uint16), vc.view(np.uint16))


def test_loose_max_context_len_changes_nothing():
    """A max_context_len several times the longest context (with block-table
    rows widened to allow it): bit-identical for a given partition size, and
    the default for the loose bound within tolerance of the oracle."""
    pa = require_gpu()
    w = W.multi_custom("loose_multi", 48, [9, 300, 1500], [3, 5, 2], 32, 8, 128, 16)
    t, kc0, vc0, q = prepare(w)
    ref = oracle_multi(w, kc0, vc0, q)
    pa.kv_append(t["k_new"], t["v_new"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    nbt = w.block_tables.shape[1]
    bt = torch.zeros((w.num_seqs, 4 * nbt), dtype=torch.int32, device="cuda")
    bt[:, :nbt] = t["block_tables"]
    loose = 4 * nbt * w.block_size

    def run(tables, maxctx, P):
        return pa.decode_multi(t["q"], t["k_cache"], t["v_cache"], tables, t["context_lens"], t["query_start"],
                               w.scale, maxctx, w.max_query_len, partition_size=P)

    for P in (-1, 64, 512):
        say("loose multi, partition", P, "max_context_len", w.max_context_len, "vs", loose)
        tight, wide = run(t["block_tables"], w.max_context_len, P), run(bt, loose, P)
        torch.cuda.synchronize()
        assert bits_equal(tight, wide), P
    out = run(bt, loose, 0)
    torch.cuda.synchronize()
    check_close(out_f64(out), ref, "bf16", "loose multi default")


@pytest.mark.parametrize("nseq", [256, 300])
def test_one_pass_order_by_length_either_side_of_the_limit(nseq):
    """One-pass launches run sequences longest first for batches of up to 256
    sequences and in batch order above that; either way every sequence gets
    its own rows.  Ragged lengths with ties; sampled sequences against the
    oracle, the rest finite."""
    pa = require_gpu()
    rng = np.random.default_rng(49 + nseq)
    lens = rng.integers(3, 700, size=nseq)
    lens[::7] = 333                                 # ties, broken by index
    news = rng.integers(1, 4, size=nseq)
    w = W.multi_custom("order_limit", 49, lens.tolist(), news.tolist(), 32, 8, 128, 16)
    t, kc0, vc0, q = prepare(w)
    seqs = sorted(set([0, 7, 14, int(np.argmax(lens)), int(np.argmin(lens)), nseq - 1] +
                      rng.choice(nseq, size=6, replace=False).tolist()))
    ref = oracle_multi(w, kc0, vc0, q, seqs=seqs)
    say("one pass order, seqs", nseq)
    out = run_gpu(pa, w, t, partition_size=-1)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(w.query_start[b], w.query_start[b + 1]) for b in seqs])
    check_close(out_f64(out)[rows], ref[rows], "bf16", f"order {nseq}")
    assert np.isfinite(out_f64(out)).all()


# Prompt chunks: many new tokens per sequence (up to all of its context, a
# whole prompt), some sequences with none, several 128-column groups.
CHUNK_LENS = [300, 1, 97, 640, 129, 1000, 512, 64]
CHUNK_NEWS = [300, 1, 0, 200, 64, 333, 17, 64]
CHUNK_SHAPES = [  # (block_size, num_heads, num_kv_heads, head_dim)
    (16, 32, 8, 128),
    (32, 32, 8, 128),
    (16, 64, 8, 128),
    (32, 16, 2, 64),
    (16, 8, 8, 64),
]


@pytest.mark.parametrize("shape", CHUNK_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_prompt_chunks_match_oracle(shape):
    """The LDS-staged kernel with causal rows: chunks that end inside a page
    (its stale tail zeroed), columns that stop inside a chunk, waves whose
    columns see nothing of a partition, one pass and split."""
    pa = require_gpu()
    bs, hq, hkv, d = shape
    assert (hq // hkv) * max(CHUNK_NEWS) >= 64
    w = W.multi_custom("prompt_chunks", 48, CHUNK_LENS, CHUNK_NEWS, hq, hkv, d, bs)
    t, kc0, vc0, q = prepare(w)
    ref = oracle_multi(w, kc0, vc0, q)
    for P in (-1, 0, 64, 256):
        t2 = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        say("prompt chunks", shape, "partition", P, w.summary())
        out = run_gpu(pa, w, t2, partition_size=P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"prompt chunks {shape} P={P}")
        again = run_gpu(pa, w, {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()},
                        partition_size=P)
        torch.cuda.synchronize()
        assert bits_equal(out, again), f"repeat {shape} P={P}"


@pytest.mark.parametrize("shape", [(16, 32, 8, 128), (32, 16, 2, 64)], ids=lambda s: "-".join(map(str, s)))
def test_prompt_chunk_fused_append(shape):
    """pa_decode_multi_append on the LDS-staged kernel (its rows stored by a
    launch of their own first) = pa_kv_append + pa_decode_multi, bit for bit
    (outputs and whole caches), and within tolerance of the oracle."""
    pa = require_gpu()
    bs, hq, hkv, d = shape
    w = W.multi_custom("prompt_chunk_fused", 49, CHUNK_LENS, CHUNK_NEWS, hq, hkv, d, bs)
    t, kc0, vc0, q = prepare(w)
    ref = oracle_multi(w, kc0, vc0, q)
    kc_ref, vc_ref = oracle.kv_append(w._k_new, w._v_new, w.append_slots, kc0, vc0, bs)
    for P in (-1, 128):
        a = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        b = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
        say("prompt chunk fused append", shape, "partition", P)
        out_a = run_gpu(pa, w, a, partition_size=P)
        out_b = pa.decode_multi(b["q"], b["k_cache"], b["v_cache"], b["block_tables"], b["context_lens"],
                                b["query_start"], w.scale, w.max_context_len, w.max_query_len, partition_size=P,
                                k_new=b["k_new"], v_new=b["v_new"])
        torch.cuda.synchronize()
        assert bits_equal(out_a, out_b), P
        assert np.array_equal(storage_np(b["k_cache"]), kc_ref), P
        assert np.array_equal(storage_np(b["v_cache"]), vc_ref), P
        check_close(out_f64(out_b), ref, "bf16", f"prompt chunk fused {shape} P={P}")
