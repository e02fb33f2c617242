"""Paged decode on the GPU against the float64 oracle.

Small workloads (the oracle takes seconds) cover every kernel family, path
(single pass, split with several partition sizes, library default), dtype,
block size, head_dim and group size, with ragged lengths around every tile
boundary.  The named full-size workloads are checked on sampled sequences in
the launch configuration the benchmark uses.  Invariants that need no oracle
(page-permutation and repeat bit-identity, stage API = one call) are checked
as well."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import (bits_equal, check_close, out_f64, report, require_gpu, run_step_updates, say,
                      step_and_reference)

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 95, 96, 97, 100, 255, 256, 257, 513, 700]

SHAPES = [  # (dtype, block_size, num_heads, num_kv_heads, head_dim)
    ("f32", 16, 4, 4, 64),
    ("f32", 32, 32, 8, 128),
    ("f32", 16, 6, 3, 128),
    ("bf16", 16, 32, 8, 128),
    ("bf16", 32, 32, 8, 128),
    ("bf16", 16, 64, 8, 128),
    ("bf16", 32, 16, 1, 64),
    ("bf16", 16, 4, 4, 64),
    ("bf16", 16, 10, 2, 128),
]
PATHS = [-1, 0, 32, 96, 512, 2048]      # 2048 on streaming loads: 12-wave workgroups


def _kernels(dtype):
    return ["valu", "mfma"] if dtype == "bf16" else ["valu"]


REUSE = ["stream", "shared"]


def run_decode(pa, w, t, kernel="auto", partition_size=None, reuse="auto"):
    ps = w.partition_size if partition_size is None else partition_size
    return pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                     w.scale, w.max_context_len, partition_size=ps, kernel=kernel, reuse=reuse)


def natural_reuse(w):
    """The load path a caller would pick: shared when sequences share pages."""
    return "shared" if w.extra.get("shared_pages") else "stream"


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_decode_small_all_paths(shape):
    pa = require_gpu()
    dtype, bs, hq, hkv, d = shape
    w = W.custom("ragged", 7, dtype, RAGGED, hq, hkv, d, bs)
    say("small", shape, w.summary())
    t = W.make_tensors(w, "cuda")
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    for kernel in _kernels(dtype):
        for reuse in REUSE:
            for ps in PATHS:
                say("  kernel", kernel, "reuse", reuse, "partition", ps)
                out = run_decode(pa, w, t, kernel, ps, reuse)
                torch.cuda.synchronize()
                check_close(out_f64(out), ref, dtype, f"{shape} {kernel} {reuse} P={ps}")


@pytest.mark.parametrize("figure", [False, True])
def test_tiny_workload(figure):
    """2 seqs of 36 and 42 tokens, fp32, D 64, 4/4 heads (one with the
    page-table figure's pages 7, 14, 2)."""
    pa = require_gpu()
    w = W.tiny(figure_table=figure)
    say("tiny", figure, w.block_tables.tolist())
    t = W.make_tensors(w, "cuda")
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    for reuse in REUSE:
        for ps in PATHS:
            out = run_decode(pa, w, t, "auto", ps, reuse)
            torch.cuda.synchronize()
            check_close(out_f64(out), ref, "f32", f"tiny {reuse} P={ps}")


def test_empty_context_gives_zeros():
    pa = require_gpu()
    w = W.custom("with_empty", 8, "bf16", [40, 1, 77, 600], 32, 8, 128, 16)
    say("empty context")
    t = W.make_tensors(w, "cuda")
    t["context_lens"][2] = 0                 # sequence 2 has nothing to attend to
    w.context_lens = w.context_lens.copy()
    w.context_lens[2] = 0
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    assert not ref[2].any()
    for kernel in ("valu", "mfma"):
        for reuse in REUSE:
            for ps in PATHS:
                out = run_decode(pa, w, t, kernel, ps, reuse)
                torch.cuda.synchronize()
                got = out_f64(out)
                assert not got[2].any()
                check_close(got, ref, "bf16", f"empty {kernel} {reuse} P={ps}")
    # every sequence empty, max_context_len 0
    t["context_lens"].zero_()
    for kernel in ("valu", "mfma"):
        for reuse in REUSE:
            for ps in (-1, 0):
                out = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                t["context_lens"], w.scale, 0, partition_size=ps, kernel=kernel,
                                reuse=reuse)
                torch.cuda.synchronize()
                assert not out_f64(out).any()


def _sample(w, n, seed):
    rng = np.random.default_rng(seed)
    order = np.argsort(w.context_lens)
    pick = {int(order[0]), int(order[-1])}
    rest = [b for b in range(w.num_seqs) if b not in pick]
    pick |= set(int(b) for b in rng.choice(rest, size=min(n - 2, len(rest)), replace=False))
    return sorted(pick)


@pytest.mark.parametrize("name", ["tiny", "llama3_8b", "llama3_70b", "prefix_share", "beam_fork",
                                  "long_context"])
def test_named_workload_full_size(name):
    """Full-size workload in the launch configuration the benchmark times
    (library-default partitions, the load path a caller would pick), every
    sequence against the oracle; the other load path and the vector-ALU
    kernel as further checks."""
    pa = require_gpu()
    w = W.by_name(name)
    say("full", name, w.summary())
    t = W.make_tensors(w, "cuda")
    seqs = list(range(w.num_seqs))
    ref = step_and_reference(pa, w, t, seqs)
    nat = natural_reuse(w)
    other = "shared" if nat == "stream" else "stream"
    for kernel, reuse in [("auto", nat), ("auto", other), ("valu", nat)]:
        out = run_decode(pa, w, t, kernel, reuse=reuse)
        torch.cuda.synchronize()
        got = out_f64(out)[seqs]
        stats = check_close(got, ref, w.dtype, f"{name} {kernel} {reuse}")
        report(f"pa_decode {name} {kernel} {reuse} ({len(seqs)} seqs)", stats)
        assert np.isfinite(out_f64(out)).all()


def test_single_pass_matches_split_at_full_size():
    pa = require_gpu()
    w = W.llama3_8b()
    say("single vs split", w.summary())
    t = W.make_tensors(w, "cuda")
    seqs = _sample(w, 6, 12)
    ref = step_and_reference(pa, w, t, seqs)
    for reuse in REUSE:
        for ps in (-1, 256, 1024):
            out = run_decode(pa, w, t, "mfma", ps, reuse)
            torch.cuda.synchronize()
            check_close(out_f64(out)[seqs], ref, "bf16", f"{reuse} P={ps}")


@pytest.mark.parametrize("kernel,ps,reuse", [("mfma", 0, "stream"), ("mfma", -1, "stream"),
                                             ("mfma", 0, "shared"), ("mfma", -1, "shared"),
                                             ("valu", 64, "stream"), ("valu", -1, "shared")])
def test_page_permutation_is_bit_identical(kernel, ps, reuse):
    """Moving physical pages (with the matching table edit) changes no bit:
    the work order depends only on logical positions."""
    pa = require_gpu()
    w = W.llama3_8b(seed=21, num_seqs=12, len_range=(1, 1500))
    say("permutation", kernel, ps, reuse)
    t = W.make_tensors(w, "cuda")
    run_step_updates(pa, w, t)
    base = run_decode(pa, w, t, kernel, ps, reuse).clone()
    perm = torch.from_numpy(np.random.default_rng(22).permutation(w.num_blocks)).cuda()
    kc2 = torch.empty_like(t["k_cache"])
    vc2 = torch.empty_like(t["v_cache"])
    kc2[perm] = t["k_cache"]
    vc2[perm] = t["v_cache"]
    tables2 = perm[t["block_tables"].long()].to(torch.int32).contiguous()
    out2 = pa.decode(t["q"], kc2, vc2, tables2, t["context_lens"], w.scale, w.max_context_len,
                     partition_size=ps, kernel=kernel, reuse=reuse)
    again = run_decode(pa, w, t, kernel, ps, reuse)
    torch.cuda.synchronize()
    assert bits_equal(out2, base)
    assert bits_equal(again, base)


def test_stage_api_equals_one_call():
    pa = require_gpu()
    w = W.llama3_70b(num_seqs=16, clip=(1, 3000))
    say("stages", w.summary())
    t = W.make_tensors(w, "cuda")
    run_step_updates(pa, w, t)
    for P, reuse in ((64, "stream"), (512, "shared")):
        one = run_decode(pa, w, t, "mfma", P, reuse)
        ws = pa.make_workspace(t["q"], w.num_kv_heads, w.max_context_len, P)
        pa.decode_partition(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                            w.scale, w.max_context_len, P, ws, kernel="mfma", reuse=reuse)
        two = torch.empty_like(one)
        pa.decode_reduce(ws, t["context_lens"], two, w.max_context_len, P)
        torch.cuda.synchronize()
        assert bits_equal(one, two)


def test_group_of_sixteen_and_head_dim_64():
    pa = require_gpu()
    w = W.custom("g16", 9, "bf16", [5, 300, 1025, 2048], 32, 2, 64, 32)
    say("g16", w.summary())
    t = W.make_tensors(w, "cuda")
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    for kernel in ("valu", "mfma"):
        for reuse in REUSE:
            for ps in (-1, 0, 128, 2048):
                out = run_decode(pa, w, t, kernel, ps, reuse)
                torch.cuda.synchronize()
                check_close(out_f64(out), ref, "bf16", f"g16 {kernel} {reuse} P={ps}")


@pytest.mark.parametrize("shape", [(16, 32, 8, 128), (32, 32, 2, 128), (32, 16, 8, 64)],
                         ids=lambda s: "-".join(map(str, s)))
def test_single_pass_over_many_pairs(shape):
    """1,024 and more (sequence, kv head) pairs with contexts past 512: the
    streaming default is one pass of 12-wave workgroups (16 query heads per
    kv head in the second shape); sampled sequences against the oracle, and
    the 4-wave split path as a cross-check."""
    pa = require_gpu()
    bs, hq, hkv, d = shape
    nseq = 1024 // hkv
    lens = np.random.default_rng(14).integers(1, 1500, size=nseq)
    lens[3] = 1500
    w = W.custom("many_pairs", 14, "bf16", lens.tolist(), hq, hkv, d, bs)
    assert pa.decode_partition_size(w.num_seqs, hkv, w.max_context_len, 0) == 0
    say("many pairs", shape, w.summary())
    t = W.make_tensors(w, "cuda")
    seqs = _sample(w, 10, 15)
    ref = step_and_reference(pa, w, t, seqs)
    for ps in (0, -1, 256):
        out = run_decode(pa, w, t, "mfma", ps, "stream")
        torch.cuda.synchronize()
        check_close(out_f64(out)[seqs], ref, "bf16", f"many pairs {shape} P={ps}")
        assert np.isfinite(out_f64(out)).all()


def test_bad_table_entries_stay_in_bounds():
    """Out-of-range page ids past the used entries are never read, and used
    out-of-range ids are clamped (output unspecified, but finite memory)."""
    pa = require_gpu()
    w = W.custom("pad", 10, "bf16", [17, 40], 32, 8, 128, 16)
    say("bad table entries")
    t = W.make_tensors(w, "cuda")
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    bt = t["block_tables"].clone()
    bt[0, 2:] = 2 ** 30          # entries past ceil(17 / 16) = 2: never read
    for reuse in REUSE:
        out = pa.decode(t["q"], t["k_cache"], t["v_cache"], bt, t["context_lens"], w.scale,
                        w.max_context_len, partition_size=0, kernel="mfma", reuse=reuse)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"padding entries {reuse}")
    bt[1, 0] = -5                # a used entry out of range: guarded, no fault
    for reuse in REUSE:
        out = pa.decode(t["q"], t["k_cache"], t["v_cache"], bt, t["context_lens"], w.scale,
                        w.max_context_len, partition_size=0, kernel="mfma", reuse=reuse)
        torch.cuda.synchronize()


def test_loose_max_context_len_changes_nothing():
    """max_context_len is only an upper bound.  A loose one (four times the
    table width, so about 16 times the longest sequence) sizes a larger grid
    whose extra partitions hold no tokens: for a given partition size every
    output bit stays the same, and the library default for the loose bound
    stays within tolerance of the oracle."""
    pa = require_gpu()
    w = W.custom("loose", 12, "bf16", [5, 300, 1025, 2000], 32, 8, 128, 16)
    say("loose max_context_len", w.summary())
    t = W.make_tensors(w, "cuda")
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    nbt = w.block_tables.shape[1]
    bt = torch.zeros((w.num_seqs, 4 * nbt), dtype=torch.int32, device="cuda")
    bt[:, :nbt] = t["block_tables"]
    loose = 4 * nbt * w.block_size
    for kernel in ("valu", "mfma"):
        for ps in (-1, 64, 512):
            say("  ", kernel, "partition", ps, "max_context_len", w.max_context_len, "vs", loose)
            tight = run_decode(pa, w, t, kernel, ps, "stream")
            wide = pa.decode(t["q"], t["k_cache"], t["v_cache"], bt, t["context_lens"], w.scale, loose,
                             partition_size=ps, kernel=kernel, reuse="stream")
            torch.cuda.synchronize()
            assert bits_equal(tight, wide), (kernel, ps)
        out = pa.decode(t["q"], t["k_cache"], t["v_cache"], bt, t["context_lens"], w.scale, loose,
                        partition_size=0, kernel=kernel)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"loose default {kernel}")


@pytest.mark.parametrize("shape", [(16, 32, 8, 128), (32, 16, 4, 64)], ids=lambda s: "-".join(map(str, s)))
def test_longest_first_one_pass(shape):
    """512 to 1,023 (sequence, kv head) pairs: one pass of 12-wave workgroups
    taking the sequences longest first.  Ragged lengths with ties and a
    sequence of length 0; bit-identical to the same one pass in batch order
    reached through a permuted batch (the order changes no bit), and sampled
    sequences against the oracle."""
    pa = require_gpu()
    bs, hq, hkv, d = shape
    nseq = 768 // hkv
    rng = np.random.default_rng(16)
    lens = rng.integers(1, 3000, size=nseq)
    lens[::5] = 1234                                 # ties
    w = W.custom("longest_first", 16, "bf16", lens.tolist(), hq, hkv, d, bs)
    assert pa.decode_partition_size(w.num_seqs, hkv, w.max_context_len, 0) == 0
    t = W.make_tensors(w, "cuda")
    t["context_lens"][2] = 0
    w.context_lens = w.context_lens.copy()
    w.context_lens[2] = 0
    seqs = sorted(set([0, 2, 5, 10, int(np.argmax(w.context_lens)), nseq - 1] +
                      rng.choice(nseq, size=6, replace=False).tolist()))
    ref = step_and_reference(pa, w, t, seqs)
    say("longest first", shape, w.summary())
    out = run_decode(pa, w, t, "mfma", 0, "stream")
    torch.cuda.synchronize()
    check_close(out_f64(out)[seqs], ref, "bf16", f"longest first {shape}")
    assert not out_f64(out)[2].any()
    # the same batch reversed: each sequence lands in another workgroup
    perm = torch.arange(nseq - 1, -1, -1, device="cuda")
    out_r = pa.decode(t["q"][perm].contiguous(), t["k_cache"], t["v_cache"], t["block_tables"][perm].contiguous(),
                      t["context_lens"][perm].contiguous(), w.scale, w.max_context_len, partition_size=0,
                      kernel="mfma", reuse="stream")
    torch.cuda.synchronize()
    assert bits_equal(out_r[perm].contiguous(), out)


@pytest.mark.parametrize("nseq", [256, 257])
def test_longest_first_limit_on_sequences(nseq):
    """512-odd pairs from 256 sequences of 2 kv heads take the longest-first
    pass; 257 sequences exceed what the kernels rank and take the split rule.
    Both against the oracle on sampled sequences, contexts ragged with ties."""
    pa = require_gpu()
    rng = np.random.default_rng(17 + nseq)
    lens = rng.integers(1, 1200, size=nseq)
    lens[::9] = 700
    lens[1] = 1200
    w = W.custom("seq_limit", 17, "bf16", lens.tolist(), 16, 2, 128, 16)
    P = pa.decode_partition_size(w.num_seqs, 2, w.max_context_len, 0)
    assert (P == 0) == (nseq == 256)
    t = W.make_tensors(w, "cuda")
    seqs = sorted(set([0, 1, 9, 18, nseq - 1] + rng.choice(nseq, size=7, replace=False).tolist()))
    ref = step_and_reference(pa, w, t, seqs)
    say("sequence limit", nseq, "partition", P)
    out = run_decode(pa, w, t, "mfma", 0, "stream")
    torch.cuda.synchronize()
    check_close(out_f64(out)[seqs], ref, "bf16", f"seq limit {nseq}")
    assert np.isfinite(out_f64(out)).all()
