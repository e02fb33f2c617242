"""pa_decode_shared_prefix on the GPU against the float64 oracle.

The shared pages are read once for many sequences' queries (a multi-query
launch whose rows all see the whole shared prefix), the rest of each context
per sequence, and the partials merged as in the split path.  The oracle is
the plain decode definition over each sequence's own block table: sharing
only changes how often a page is read, never the result.

Shared-prefix batches of any head shape are built from independent ragged
sequences by pointing every row's leading table entries at row 0's pages (the
oracle reads through the same tables, so both sides see the same bytes); the
named prefix-sharing and beam workloads are checked at full size."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bits_equal, check_close, out_f64, require_gpu, say, step_and_reference, storage_np

pytestmark = pytest.mark.gpu


def _share_rows(w, t, shared_tokens):
    """Make every sequence read row 0's pages for its first shared_tokens
    positions (whole pages), on the host copy and the device copy alike."""
    n = shared_tokens // w.block_size
    tables = w.block_tables.copy()
    tables[:, :n] = tables[0, :n]
    w.block_tables = tables
    t["block_tables"].copy_(torch.from_numpy(tables))


def _shared_batch(name, seed, hq, hkv, d, bs, shared_tokens, nseq=24):
    rng = np.random.default_rng(seed)
    lens = shared_tokens + 2 + rng.integers(0, 400, size=nseq)
    lens[min(1, nseq - 1)] = shared_tokens + 2      # the shortest context allowed
    w = W.custom(name, seed, "bf16", lens.tolist(), hq, hkv, d, bs)
    t = W.make_tensors(w, "cuda")
    _share_rows(w, t, shared_tokens)
    return w, t


def _run(pa, w, t, shared_len, P):
    return pa.decode_shared_prefix(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                   w.scale, w.max_context_len, shared_len, P)


SHAPES = [  # (num_heads, num_kv_heads, head_dim, block_size)
    (32, 8, 128, 16),
    (32, 8, 128, 32),
    (64, 8, 128, 16),     # G = 8: 4 sequences per 32-column group
    (32, 2, 64, 16),      # G = 16: 2 sequences per group, D 64
    (32, 2, 64, 32),      # the same at block 32
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_shared_prefix_matches_oracle(shape):
    pa = require_gpu()
    hq, hkv, d, bs = shape
    w, t = _shared_batch("shared", 41, hq, hkv, d, bs, shared_tokens=640)
    say("shared prefix", shape, w.summary())
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    S = pa.shared_prefix_len(w.block_tables, w.context_lens, bs)
    assert S == 640
    for P in (32, 64, 128, 256, 96):
        # the whole shared run, and shorter ones (still valid: fewer shared
        # pages), ending on and inside partitions (the extra slot)
        for s_len in sorted({S, S - bs, max(S - P - bs, 0), bs}, reverse=True):
            say("  partition", P, "shared_len", s_len, "ends inside a partition:", s_len % P != 0)
            out = _run(pa, w, t, s_len, P)
            torch.cuda.synchronize()
            check_close(out_f64(out), ref, "bf16", f"shared {shape} P={P} S={s_len}")
        again = _run(pa, w, t, S - bs, P)
        torch.cuda.synchronize()
        assert bits_equal(_run(pa, w, t, S - bs, P), again), f"repeat {shape} P={P}"


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_shared_prefix_negative_and_zero_scale(scale):
    """The wide prefix launch folds the scale's sign into the queries and
    scales the column max: a negative scale and a zero scale (uniform
    weights over every position) against the oracle, shared length ending
    inside a 64-token chunk."""
    pa = require_gpu()
    w, t = _shared_batch("shared_scale", 45, 32, 8, 128, 32, shared_tokens=672, nseq=20)
    S = pa.shared_prefix_len(w.block_tables, w.context_lens, 32)
    assert S == 672 and 4 * w.num_seqs >= 64
    say("shared prefix scale", scale, w.summary())
    ref = step_and_reference(pa, w, t, range(w.num_seqs), scale=np.float32(scale))
    for P in (64, 256):
        out = pa.decode_shared_prefix(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                      float(np.float32(scale)), w.max_context_len, S, P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"shared scale {scale} P={P}")


def test_zero_shared_length_is_the_split_path():
    """shared_len 0 launches no prefix work: bit-identical to pa_decode's
    split path on the matrix-core kernel with shared-page loads (only the
    workspace rows are one slot longer)."""
    pa = require_gpu()
    w, t = _shared_batch("shared_zero", 42, 32, 8, 128, 16, shared_tokens=320)
    say("shared prefix, shared_len 0", w.summary())
    step_and_reference(pa, w, t, [0])
    for P in (64, 256):
        one = _run(pa, w, t, 0, P)
        two = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"], w.scale,
                        w.max_context_len, partition_size=P, kernel="mfma", reuse="shared")
        torch.cuda.synchronize()
        assert bits_equal(one, two), P


def test_many_sequences_fill_several_column_groups():
    """200 sequences x 4 heads = 800 columns: 25 column groups of 32 over the
    prefix; sampled sequences against the oracle."""
    pa = require_gpu()
    w, t = _shared_batch("shared_many", 43, 32, 8, 128, 16, shared_tokens=1024, nseq=200)
    say("shared prefix, 200 sequences", w.summary())
    seqs = [0, 1, 7, 31, 32, 33, 99, 150, 198, 199]
    ref = step_and_reference(pa, w, t, seqs)
    S = pa.shared_prefix_len(w.block_tables, w.context_lens, 16)
    assert S == 1024
    for P in (256, 384):                              # 1024 = 2 x 384 + 256: the extra slot
        out = _run(pa, w, t, S, P)
        torch.cuda.synchronize()
        check_close(out_f64(out)[seqs], ref, "bf16", f"shared 200 seqs P={P}")


@pytest.mark.parametrize("name", ["prefix_share", "beam_fork"])
def test_named_workload_full_size(name):
    """The 100 x 10,000-token prefix batch and the 8 beams over a 32,768-token
    prompt, after the step's copy-on-write copies and appends, with the shared
    length the block tables give at partition 2048; sampled sequences against
    the oracle."""
    pa = require_gpu()
    w = W.by_name(name)
    say("shared prefix full", name, w.summary())
    t = W.make_tensors(w, "cuda")
    rng = np.random.default_rng(23)
    order = np.argsort(w.context_lens)
    seqs = sorted({int(order[0]), int(order[-1])} |
                  set(int(s) for s in rng.choice(w.num_seqs, size=min(6, w.num_seqs), replace=False)))
    ref = step_and_reference(pa, w, t, seqs)
    S = pa.shared_prefix_len(w.block_tables, w.context_lens, w.block_size)
    say("  shared_len", S)
    assert S >= 9984
    for P in (1024, 2048, 0):                        # 0: the library default
        out = _run(pa, w, t, S, P)
        torch.cuda.synchronize()
        stats = check_close(out_f64(out)[seqs], ref, "bf16", f"shared {name} P={P}")
        say("  ", P, stats)


def test_fused_append():
    """Each sequence's newest rows appended by the partition kernel of the
    shared-prefix call (position L - 1 lies past the shared prefix): caches bit
    for bit against the oracle's append, output within tolerance of the oracle
    and bit-identical to pa_kv_append followed by the same call without rows."""
    pa = require_gpu()
    w, t = _shared_batch("shared_fused", 44, 32, 8, 128, 16, shared_tokens=512)
    say("shared prefix, fused append", w.summary())
    B = w.num_seqs
    assert sorted(w.append_seq.tolist()) == list(range(B))
    k_new = torch.zeros(B, w.num_kv_heads, w.head_dim, dtype=t["k_new"].dtype, device="cuda")
    v_new = torch.zeros_like(k_new)
    mask = np.full(B, -1, dtype=np.int64)
    for i, b in enumerate(w.append_seq.tolist()):
        k_new[b] = t["k_new"][i]
        v_new[b] = t["v_new"][i]
        mask[b] = w.append_slots[i]
    kc0, vc0 = storage_np(t["k_cache"]), storage_np(t["v_cache"])
    rk, rv = oracle.kv_append(storage_np(k_new), storage_np(v_new), mask, kc0, vc0, w.block_size)
    ref = oracle.decode(storage_np(t["q"]), rk, rv, w.block_tables, w.context_lens, w.scale, w.block_size,
                        "bf16")
    slots = torch.from_numpy(mask).cuda()
    S = pa.shared_prefix_len(w.block_tables, w.context_lens, w.block_size)
    assert S == 512
    for P in (64, 256, 192):                          # 512 = 2 x 192 + 128: the extra slot
        say("  partition", P, "shared_len", S)
        kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
        out = pa.decode_shared_prefix(t["q"], kc, vc, t["block_tables"], t["context_lens"], w.scale,
                                      w.max_context_len, S, P, k_new=k_new, v_new=v_new, slot_mapping=slots)
        torch.cuda.synchronize()
        assert np.array_equal(storage_np(kc).view(np.uint16), rk.view(np.uint16))
        assert np.array_equal(storage_np(vc).view(np.uint16), rv.view(np.uint16))
        check_close(out_f64(out), ref, "bf16", f"shared fused P={P}")
        kc2, vc2 = t["k_cache"].clone(), t["v_cache"].clone()
        pa.kv_append(k_new, v_new, slots, kc2, vc2)
        out2 = pa.decode_shared_prefix(t["q"], kc2, vc2, t["block_tables"], t["context_lens"], w.scale,
                                       w.max_context_len, S, P)
        torch.cuda.synchronize()
        assert bits_equal(out, out2), f"fused != separate P={P}"


@pytest.mark.parametrize("shape", [(32, 8, 128, 16), (32, 8, 64, 32)], ids=lambda s: "-".join(map(str, s)))
@pytest.mark.parametrize("nseq", [12, 8, 4, 1])
def test_few_sequences(nseq, shape):
    """Fewer than 64 columns per kv head: the multi-query prefix stage.  12
    sequences x 4 heads = 48 columns run two 16-column tiles per workgroup
    over two groups; 8 fill one group of 32 columns (the prefix stage then
    runs one tile per workgroup over two groups), 4 fit one tile, and a
    single sequence shares a prefix with itself.  D 128 at block 16 and D 64
    at block 32."""
    pa = require_gpu()
    hq, hkv, d, bs = shape
    w, t = _shared_batch("shared_few", 45 + nseq, hq, hkv, d, bs, shared_tokens=768, nseq=nseq)
    say("shared prefix,", nseq, "sequences", shape, w.summary())
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    S = pa.shared_prefix_len(w.block_tables, w.context_lens, bs)
    assert S == 768
    for P in (128, 256, 320):                         # 768 = 2 x 320 + 128: the extra slot
        out = _run(pa, w, t, S, P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"shared {nseq} seqs {shape} P={P}")


@pytest.mark.parametrize("nseq", [24, 8])
def test_sequences_ending_at_the_prefix(nseq):
    """Sequences whose whole context is the shared prefix (their rest-of-
    context work is empty: no positions, an empty partial) beside longer
    ones, and a batch in which every sequence ends there (at P = 64 no rest
    workgroup is launched at all); the LDS-staged prefix stage (24 sequences
    x 4 heads) and the multi-query one (8)."""
    pa = require_gpu()
    S = 640
    rng = np.random.default_rng(60 + nseq)
    lens = S + 2 + rng.integers(0, 300, size=nseq)
    lens[1::3] = S                                    # every third sequence ends at the prefix
    for every in (False, True):
        L = np.full(nseq, S) if every else lens
        w = W.custom("shared_end", 61 + nseq, "bf16", L.tolist(), 32, 8, 128, 16)
        t = W.make_tensors(w, "cuda")
        _share_rows(w, t, S)
        say("shared prefix, sequences ending at it", nseq, "every one" if every else "every third", w.summary())
        ref = step_and_reference(pa, w, t, range(nseq))
        assert pa.shared_prefix_len(w.block_tables, w.context_lens, 16) == S
        for P in (64, 256, 0):
            out = _run(pa, w, t, S, P)
            torch.cuda.synchronize()
            check_close(out_f64(out), ref, "bf16", f"ending at the prefix {nseq} every={every} P={P}")


def test_largest_batch():
    """1,024 sequences, the most one call takes: 4,096 (sequence, head)
    columns in 128 groups over the shared prefix; sampled sequences, the
    first and last column groups included."""
    pa = require_gpu()
    w, t = _shared_batch("shared_max", 47, 32, 8, 128, 16, shared_tokens=96, nseq=1024)
    say("shared prefix, 1,024 sequences", w.summary())
    seqs = [0, 1, 2, 7, 8, 511, 512, 1015, 1016, 1023]
    ref = step_and_reference(pa, w, t, seqs)
    S = pa.shared_prefix_len(w.block_tables, w.context_lens, 16)
    assert S == 96
    for P in (64, 256):
        out = _run(pa, w, t, S, P)
        torch.cuda.synchronize()
        check_close(out_f64(out)[seqs], ref, "bf16", f"shared 1024 seqs P={P}")


def _grouped_batch(seed, hq, hkv, d, bs, groups, loner_len=300):
    """Sequences in groups [(size, shared_tokens)], then one sequence in no
    group; each group's rows point their leading entries at its first row's
    pages.  A group with 0 shared tokens shares nothing (several sequences
    read one by one, as the block manager reports sequences between two
    sharing runs); max_group_size bounds only the groups that share."""
    rng = np.random.default_rng(seed)
    lens, shared = [], []
    for size, S in groups:
        for _ in range(size):
            lens.append(S + 2 + int(rng.integers(0, 300)))
            shared.append(S)
    lens.append(loner_len)
    shared.append(0)
    w = W.custom("groups", seed, "bf16", lens, hq, hkv, d, bs)
    t = W.make_tensors(w, "cuda")
    tables = w.block_tables.copy()
    start, starts = 0, [0]
    for size, S in groups:
        tables[start:start + size, :S // bs] = tables[start, :S // bs]
        start += size
        starts.append(start)
    w.block_tables = tables
    t["block_tables"].copy_(torch.from_numpy(tables))
    arrays = dict(group_start=torch.tensor(starts, dtype=torch.int32, device="cuda"),
                  group_shared_len=torch.tensor([S for _, S in groups], dtype=torch.int32, device="cuda"),
                  seq_shared_len=torch.tensor(shared, dtype=torch.int32, device="cuda"),
                  max_group_size=max([size for size, S in groups if S > 0] + [1]),
                  max_shared_len=max(S for _, S in groups))
    return w, t, arrays


@pytest.mark.parametrize("shape", [(32, 8, 128, 16), (64, 8, 128, 32), (32, 8, 128, 32), (32, 8, 64, 16)],
                         ids=lambda s: "-".join(map(str, s)))
def test_prefix_groups_match_oracle(shape):
    """Groups of 10, 5, 1 and 14 sequences, three sequences sharing nothing
    between the second and third, and one sequence in no group.  At block 16
    the shared lengths 336 and 208 end in the middle of a 32-token chunk and
    of a partition; at block 32, 320 and 480 end on or inside partitions.
    With 4 heads per kv head the groups have up to 56 columns: the
    multi-query prefix stage with two 16-column tiles per workgroup (D 128
    and 64, block 16 and 32); with 8, the LDS-staged stage."""
    pa = require_gpu()
    hq, hkv, d, bs = shape
    groups = ([(10, 336), (5, 96), (3, 0), (1, 640), (14, 208)] if bs == 16 else
              [(10, 320), (5, 96), (3, 0), (1, 640), (14, 480)])
    w, t, arr = _grouped_batch(48, hq, hkv, d, bs, groups)
    say("prefix groups", shape, groups, w.summary())
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    for P in (64, 256, 0):
        out = pa.decode_shared_prefix_groups(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                             t["context_lens"], w.scale, w.max_context_len, partition_size=P, **arr)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"groups {shape} P={P}")


@pytest.mark.parametrize("bs", [16, 32])
def test_prefix_groups_wide_match_oracle(bs):
    """Groups of 20, 17 and 16 sequences x 4 heads (64 to 80 columns per kv
    head): the LDS-staged prefix kernel with partitions of its own, each
    sequence's slot shift from its shared length (336 and 208 end inside a
    64-token chunk at block 16), three sequences sharing nothing between the
    groups and one in no group; with and without the fused append."""
    pa = require_gpu()
    groups = ([(20, 336), (3, 0), (17, 208), (16, 640)] if bs == 16 else
              [(20, 320), (3, 0), (17, 224), (16, 640)])
    w, t, arr = _grouped_batch(52 + bs, 32, 8, 128, bs, groups)
    assert 4 * arr["max_group_size"] >= 64
    say("prefix groups, wide", bs, groups, w.summary())
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    for P in (64, 256, 0):
        out = pa.decode_shared_prefix_groups(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                             t["context_lens"], w.scale, w.max_context_len, partition_size=P, **arr)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"groups wide bs {bs} P={P}")
    B = w.num_seqs
    k_new = torch.zeros(B, w.num_kv_heads, w.head_dim, dtype=t["k_new"].dtype, device="cuda")
    v_new = torch.zeros_like(k_new)
    mask = np.full(B, -1, dtype=np.int64)
    for i, b in enumerate(w.append_seq.tolist()):
        k_new[b] = t["k_new"][i]
        v_new[b] = t["v_new"][i]
        mask[b] = w.append_slots[i]
    kc0, vc0 = storage_np(t["k_cache"]), storage_np(t["v_cache"])
    rk, rv = oracle.kv_append(storage_np(k_new), storage_np(v_new), mask, kc0, vc0, w.block_size)
    ref2 = oracle.decode(storage_np(t["q"]), rk, rv, w.block_tables, w.context_lens, w.scale, w.block_size,
                         "bf16")
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    out = pa.decode_shared_prefix_groups(t["q"], kc, vc, t["block_tables"], t["context_lens"], w.scale,
                                         w.max_context_len, partition_size=0, k_new=k_new, v_new=v_new,
                                         slot_mapping=torch.from_numpy(mask).cuda(), **arr)
    torch.cuda.synchronize()
    assert np.array_equal(storage_np(kc).view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(storage_np(vc).view(np.uint16), rv.view(np.uint16))
    check_close(out_f64(out), ref2, "bf16", f"groups wide fused bs {bs}")


def test_prefix_groups_fused_append():
    pa = require_gpu()
    w, t, arr = _grouped_batch(49, 32, 8, 128, 16, [(6, 256), (7, 160)])
    say("prefix groups, fused append", w.summary())
    B = w.num_seqs
    k_new = torch.zeros(B, w.num_kv_heads, w.head_dim, dtype=t["k_new"].dtype, device="cuda")
    v_new = torch.zeros_like(k_new)
    mask = np.full(B, -1, dtype=np.int64)
    for i, b in enumerate(w.append_seq.tolist()):
        k_new[b] = t["k_new"][i]
        v_new[b] = t["v_new"][i]
        mask[b] = w.append_slots[i]
    kc0, vc0 = storage_np(t["k_cache"]), storage_np(t["v_cache"])
    rk, rv = oracle.kv_append(storage_np(k_new), storage_np(v_new), mask, kc0, vc0, w.block_size)
    ref = oracle.decode(storage_np(t["q"]), rk, rv, w.block_tables, w.context_lens, w.scale, w.block_size,
                        "bf16")
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    out = pa.decode_shared_prefix_groups(t["q"], kc, vc, t["block_tables"], t["context_lens"], w.scale,
                                         w.max_context_len, partition_size=96, k_new=k_new, v_new=v_new,
                                         slot_mapping=torch.from_numpy(mask).cuda(), **arr)
    torch.cuda.synchronize()
    assert np.array_equal(storage_np(kc).view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(storage_np(vc).view(np.uint16), rv.view(np.uint16))
    check_close(out_f64(out), ref, "bf16", "groups fused")


def test_prefix_groups_workload_full_size():
    """Four 4,096-token prompts, each forked to 25 sequences with suffixes:
    the grouped call with each group's shared length from its tables; sampled
    sequences from every group against the oracle."""
    pa = require_gpu()
    w = W.by_name("prefix_groups")
    say("prefix groups full", w.summary())
    t = W.make_tensors(w, "cuda")
    groups = w.extra["groups"]
    seqs = sorted({a for a, _ in groups} | {a + n - 1 for a, n in groups} | {37, 61})
    ref = step_and_reference(pa, w, t, seqs)
    gsl = [pa.shared_prefix_len(w.block_tables[a:a + n], w.context_lens[a:a + n], w.block_size) for a, n in groups]
    assert gsl == [4096] * 4
    seq_sl = np.zeros(w.num_seqs, dtype=np.int32)
    for (a, n), S in zip(groups, gsl):
        seq_sl[a:a + n] = S
    arr = dict(group_start=torch.tensor([a for a, _ in groups] + [w.num_seqs], dtype=torch.int32, device="cuda"),
               group_shared_len=torch.tensor(gsl, dtype=torch.int32, device="cuda"),
               seq_shared_len=torch.from_numpy(seq_sl).cuda(), max_group_size=25, max_shared_len=4096)
    out = pa.decode_shared_prefix_groups(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                         w.scale, w.max_context_len, **arr)
    torch.cuda.synchronize()
    stats = check_close(out_f64(out)[seqs], ref, "bf16", "prefix groups full")
    say("  ", stats)
