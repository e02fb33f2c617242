"""pa_decode_append (append of each sequence's newest token fused into the
decode) on the GPU.

Three checks on every case: the caches afterwards are bit-identical to the
oracle's append of the newest rows (whole caches, NaN poison included); the
output is within tolerance of the float64 oracle decode over those caches;
and cache and output are bit-identical to the separate pa_kv_append +
pa_decode calls."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bits_equal, check_close, out_f64, reference_after_step, report, require_gpu, say, storage_np

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 97, 255, 256, 257, 513, 700]

SHAPES = [  # (dtype, block_size, num_heads, num_kv_heads, head_dim)
    ("f32", 16, 4, 4, 64),
    ("f32", 32, 32, 8, 128),
    ("bf16", 16, 32, 8, 128),
    ("bf16", 32, 32, 8, 128),
    ("bf16", 16, 64, 8, 128),
    ("bf16", 16, 16, 1, 64),
]
PATHS = [-1, 0, 64, 512]


def _kernels(dtype):
    return ["valu", "mfma"] if dtype == "bf16" else ["valu"]


def _view(dtype):
    return np.uint16 if dtype == "bf16" else np.uint32


def newest_rows(w, t):
    """Each sequence's newest appended row (k, v as [B, Hkv, D]) and the
    append mask (its slot, or -1 when the sequence appends nothing), plus the
    indices of the other appended tokens (appended beforehand, separately)."""
    B = w.num_seqs
    newest = {}
    for i, b in enumerate(w.append_seq.tolist()):
        newest[b] = i
    older = [i for i in range(len(w.append_seq)) if i not in set(newest.values())]
    k = torch.zeros(B, w.num_kv_heads, w.head_dim, dtype=t["k_new"].dtype, device="cuda")
    v = torch.zeros_like(k)
    mask = np.full(B, -1, dtype=np.int64)
    for b, i in newest.items():
        k[b] = t["k_new"][i]
        v[b] = t["v_new"][i]
        mask[b] = w.append_slots[i]
    return k, v, mask, older


def _apply_older(pa, w, t, older):
    if older:
        idx = torch.tensor(older, dtype=torch.long, device="cuda")
        pa.kv_append(t["k_new"].index_select(0, idx).contiguous(),
                     t["v_new"].index_select(0, idx).contiguous(),
                     t["slot_mapping"].index_select(0, idx).contiguous(), t["k_cache"], t["v_cache"])


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_fused_matches_oracle_and_separate_calls(shape):
    pa = require_gpu()
    dtype, bs, hq, hkv, d = shape
    w = W.custom("ragged_fused", 17, dtype, RAGGED, hq, hkv, d, bs)
    say("fused", shape, w.summary())
    t = W.make_tensors(w, "cuda")
    k_new, v_new, mask, older = newest_rows(w, t)
    assert not older and (mask >= 0).all()
    kc0, vc0 = storage_np(t["k_cache"]), storage_np(t["v_cache"])
    rk, rv = oracle.kv_append(storage_np(k_new), storage_np(v_new), mask, kc0, vc0, bs)
    q = storage_np(t["q"])
    ref = oracle.decode(q, rk, rv, w.block_tables, w.context_lens, w.scale, bs, dtype)
    view = _view(dtype)
    for kernel in _kernels(dtype):
        for reuse in ("stream", "shared"):
            for ps in PATHS:
                say("  ", kernel, reuse, ps)
                kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
                out = pa.decode_append(k_new, v_new, t["q"], kc, vc, t["block_tables"],
                                       t["context_lens"], w.scale, w.max_context_len,
                                       partition_size=ps, kernel=kernel, reuse=reuse)
                torch.cuda.synchronize()
                assert np.array_equal(storage_np(kc).view(view), rk.view(view))
                assert np.array_equal(storage_np(vc).view(view), rv.view(view))
                check_close(out_f64(out), ref, dtype, f"fused {shape} {kernel} {reuse} P={ps}")
                kc2, vc2 = t["k_cache"].clone(), t["v_cache"].clone()
                slots = torch.from_numpy(mask).cuda()
                pa.kv_append(k_new, v_new, slots, kc2, vc2)
                out2 = pa.decode(t["q"], kc2, vc2, t["block_tables"], t["context_lens"], w.scale,
                                 w.max_context_len, partition_size=ps, kernel=kernel, reuse=reuse)
                torch.cuda.synchronize()
                assert bits_equal(out, out2), f"fused != separate {shape} {kernel} {reuse} P={ps}"


def test_fused_mask_and_empty_contexts():
    """A negative slot_mapping entry: that sequence appends nothing (its
    newest row was appended earlier; the garbage row handed in must not be
    written).  L = 0: nothing appended, zeros out."""
    pa = require_gpu()
    w = W.custom("fused_mask", 18, "bf16", [40, 1, 77, 600, 33], 32, 8, 128, 16)
    say("fused mask", w.summary())
    t = W.make_tensors(w, "cuda")
    k_new, v_new, mask, _ = newest_rows(w, t)
    skip = [1, 3]
    # sequences 1 and 3 got their newest token before; hand in other rows now
    kc0, vc0 = oracle.kv_append(storage_np(k_new[skip]), storage_np(v_new[skip]), mask[skip],
                                storage_np(t["k_cache"]), storage_np(t["v_cache"]), 16)
    pa.kv_append(k_new[skip].contiguous(), v_new[skip].contiguous(),
                 torch.from_numpy(mask[skip]).cuda(), t["k_cache"], t["v_cache"])
    appending = mask.copy()
    appending[skip] = -1
    k_in, v_in = k_new.clone(), v_new.clone()
    k_in[skip] = 7.0
    v_in[skip] = -7.0
    lens = w.context_lens.copy()
    lens[4] = 0                                   # sequence 4: empty context, appends nothing
    t["context_lens"][4] = 0
    written = appending.copy()
    written[4] = -1
    rk, rv = oracle.kv_append(storage_np(k_new), storage_np(v_new), written, kc0, vc0, 16)
    ref = oracle.decode(storage_np(t["q"]), rk, rv, w.block_tables, lens, w.scale, 16, "bf16")
    assert not ref[4].any()
    for kernel in ("valu", "mfma"):
        for ps in (-1, 0, 64):
            kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
            out = pa.decode_append(k_in, v_in, t["q"], kc, vc, t["block_tables"], t["context_lens"],
                                   w.scale, w.max_context_len,
                                   slot_mapping=torch.from_numpy(appending).cuda(),
                                   partition_size=ps, kernel=kernel)
            torch.cuda.synchronize()
            assert np.array_equal(storage_np(kc).view(np.uint16), rk.view(np.uint16))
            assert np.array_equal(storage_np(vc).view(np.uint16), rv.view(np.uint16))
            got = out_f64(out)
            assert not got[4].any()
            check_close(got, ref, "bf16", f"mask {kernel} P={ps}")


# the 8B-shaped batch on 32-token pages: the streaming path's interleaved
# token order (one page per chunk) under the longest-first single pass
_BUILDERS = {"llama3_8b_bs32": lambda: W.llama3_8b(block_size=32)}


@pytest.mark.parametrize("name", ["llama3_8b", "llama3_70b", "prefix_share", "beam_fork",
                                  "long_context", "llama3_8b_bs32"])
def test_fused_named_workload_full_size(name):
    """The decode step as the benchmark runs it: set-up appends every token
    but each sequence's newest, then one pa_decode_append with the library's
    default partition and the load path a caller would pick; every sequence
    of the batch against the oracle (whole batch and each (sequence, head)
    row on its own), appended slots checked bit for bit."""
    pa = require_gpu()
    w = _BUILDERS[name]() if name in _BUILDERS else W.by_name(name)
    say("fused full", name, w.summary())
    t = W.make_tensors(w, "cuda")
    seqs = list(range(w.num_seqs))
    ref = reference_after_step(w, t, seqs)         # every row of the step appended, by the oracle
    if len(w.copy_pairs):
        pa.copy_blocks(t["k_cache"], t["v_cache"], t["copy_pairs"])
    k_new, v_new, mask, older = newest_rows(w, t)
    _apply_older(pa, w, t, older)
    reuse = "shared" if w.extra.get("shared_pages") else "stream"
    out = pa.decode_append(k_new, v_new, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                           t["context_lens"], w.scale, w.max_context_len,
                           slot_mapping=torch.from_numpy(mask).cuda(),
                           partition_size=w.partition_size, reuse=reuse)
    torch.cuda.synchronize()
    # every appended slot holds its row, bit for bit
    bs, x = w.block_size, w.x
    kc, vc = t["k_cache"], t["v_cache"]
    for b in np.flatnonzero(mask >= 0):
        page, off = divmod(int(mask[b]), bs)
        got_k = kc[page, :, :, off, :].reshape(w.num_kv_heads, w.head_dim)
        got_v = vc[page, :, :, off]
        assert bits_equal(got_k.contiguous(), k_new[b].contiguous())
        assert bits_equal(got_v.contiguous(), v_new[b].contiguous())
    stats = check_close(out_f64(out)[seqs], ref, w.dtype, f"fused {name}")
    report(f"bench step {name} ({len(seqs)} of {w.num_seqs} seqs, pa_decode_append, {reuse})", stats)


def test_fused_append_skips_a_page_outside_the_pool():
    """pa_decode_append with a block-table entry outside the pool at a
    sequence's newest position writes nothing for that sequence (the clamped
    page 0 stays as it was); every other newest row lands as the oracle puts
    it."""
    pa = require_gpu()
    w = W.custom("bad_page", 18, "bf16", [40, 70, 20, 33], 32, 8, 128, 16)
    t = W.make_tensors(w, "cuda")
    k_new, v_new, mask, older = newest_rows(w, t)
    kc0, vc0 = storage_np(t["k_cache"]), storage_np(t["v_cache"])
    tables = w.block_tables.copy()
    bad = 1
    tables[bad, (int(w.context_lens[bad]) - 1) // 16] = w.num_blocks + 7
    say("decode_append, page outside the pool")
    pa.decode_append(k_new, v_new, t["q"], t["k_cache"], t["v_cache"], torch.from_numpy(tables).cuda(),
                     t["context_lens"], w.scale, w.max_context_len, partition_size=-1)
    torch.cuda.synchronize()
    keep = np.arange(w.num_seqs) != bad
    rk, rv = oracle.kv_append(storage_np(k_new)[keep], storage_np(v_new)[keep], mask[keep], kc0, vc0, 16)
    assert np.array_equal(storage_np(t["k_cache"]).view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(storage_np(t["v_cache"]).view(np.uint16), rv.view(np.uint16))


def test_one_pass_of_wide_workgroups_appends_in_its_own_launch():
    """1,024 (sequence, kv head) pairs with contexts past 512: the default is
    one pass of 12-wave workgroups, where pa_decode_append stores the rows in
    a launch of its own first.  Caches bit-identical to the oracle's append
    (masked and empty sequences included), output bit-identical to
    pa_kv_append + pa_decode, sampled rows within tolerance of the oracle."""
    pa = require_gpu()
    rng = np.random.default_rng(23)
    lens = rng.integers(1, 1400, size=128)
    lens[5] = 1400
    w = W.custom("wide_fused", 23, "bf16", lens.tolist(), 32, 8, 128, 16)
    assert pa.decode_partition_size(w.num_seqs, 8, w.max_context_len, 0) == 0
    t = W.make_tensors(w, "cuda")
    k_new, v_new, mask, older = newest_rows(w, t)
    assert not older
    skip = [7, 40]                                  # appended earlier: nothing to append this step
    kc0, vc0 = oracle.kv_append(storage_np(k_new[skip]), storage_np(v_new[skip]), mask[skip],
                                storage_np(t["k_cache"]), storage_np(t["v_cache"]), 16)
    pa.kv_append(k_new[skip].contiguous(), v_new[skip].contiguous(), torch.from_numpy(mask[skip]).cuda(),
                 t["k_cache"], t["v_cache"])
    mask[skip] = -1
    t["context_lens"][9] = 0                        # and this one has no context at all
    lens_host = w.context_lens.copy()
    lens_host[9] = 0
    written = mask.copy()
    written[9] = -1
    rk, rv = oracle.kv_append(storage_np(k_new), storage_np(v_new), written, kc0, vc0, 16)
    seqs = [0, 5, 7, 9, 40, 77, 127]
    ref = oracle.decode(storage_np(t["q"])[seqs], rk, rv, w.block_tables[seqs], lens_host[seqs], w.scale, 16,
                        "bf16")
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    say("one pass of wide workgroups, fused append")
    out = pa.decode_append(k_new, v_new, t["q"], kc, vc, t["block_tables"], t["context_lens"], w.scale,
                           w.max_context_len, slot_mapping=torch.from_numpy(mask).cuda(), reuse="stream")
    torch.cuda.synchronize()
    assert np.array_equal(storage_np(kc).view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(storage_np(vc).view(np.uint16), rv.view(np.uint16))
    check_close(out_f64(out)[seqs], ref, "bf16", "wide one pass fused")
    assert not out_f64(out)[9].any()
    kc2, vc2 = t["k_cache"].clone(), t["v_cache"].clone()
    sel = np.flatnonzero(written >= 0)
    idx = torch.from_numpy(sel).cuda()
    pa.kv_append(k_new.index_select(0, idx).contiguous(), v_new.index_select(0, idx).contiguous(),
                 torch.from_numpy(written[sel]).cuda(), kc2, vc2)
    out2 = pa.decode(t["q"], kc2, vc2, t["block_tables"], t["context_lens"], w.scale, w.max_context_len,
                     reuse="stream")
    torch.cuda.synchronize()
    assert bits_equal(out, out2)
