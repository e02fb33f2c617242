"""KV-append scatter and page copy on the GPU: bit-exact against the oracle,
whole caches compared bit by bit (NaN poison included)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bits_equal, require_gpu, run_step_updates, say, storage_np

pytestmark = pytest.mark.gpu

SHAPES = [("f32", 16, 64), ("f32", 32, 128), ("bf16", 16, 128), ("bf16", 32, 128), ("bf16", 16, 64),
          ("bf16", 32, 64)]


def _random_cache(shape_k, shape_v, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    td = W.torch_dtype(dtype)
    kc = torch.randn(*shape_k, generator=g, device="cuda").to(td)
    vc = torch.randn(*shape_v, generator=g, device="cuda").to(td)
    # sprinkle NaN so payload preservation is exercised
    kc.view(-1)[::97] = float("nan")
    vc.view(-1)[::89] = float("nan")
    return kc, vc


@pytest.mark.parametrize("dtype,bs,d", SHAPES)
def test_append_bit_exact(dtype, bs, d):
    pa = require_gpu()
    say("append", dtype, bs, d)
    nb, hkv, T = 37, 4, 60
    x = W.chunk_elems(dtype)
    kc, vc = _random_cache((nb, hkv, d // x, bs, x), (nb, hkv, d, bs), dtype, 1)
    rng = np.random.default_rng(2)
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[[3, 17]] = -1                        # padding tokens: no write
    slots[25] = nb * bs + 7                    # out of range: skipped by the guard
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    td = W.torch_dtype(dtype)
    k = torch.randn(T, hkv, d, generator=g, device="cuda").to(td)
    v = torch.randn(T, hkv, d, generator=g, device="cuda").to(td)
    k_before, v_before = storage_np(kc), storage_np(vc)
    pa.kv_append(k, v, torch.from_numpy(slots).cuda(), kc, vc)
    torch.cuda.synchronize()
    ref_slots = slots.copy()
    ref_slots[25] = -1
    rk, rv = oracle.kv_append(storage_np(k), storage_np(v), ref_slots, k_before, v_before, bs)
    got_k, got_v = storage_np(kc), storage_np(vc)
    view = np.uint16 if dtype == "bf16" else np.uint32
    assert np.array_equal(got_k.view(view), rk.view(view))
    assert np.array_equal(got_v.view(view), rv.view(view))


@pytest.mark.parametrize("dtype,bs,d", SHAPES)
def test_bulk_append_bit_exact(dtype, bs, d):
    """A prefill-sized append (the LDS-staged kernel, 1,500 tokens: 23 full
    token groups and a ragged one): runs of consecutive slots that start and
    end mid-page, padding, out-of-range slots and a stretch of tokens
    scattered over pages, so both store orders run; whole caches against
    the oracle, bit for bit."""
    pa = require_gpu()
    say("bulk append", dtype, bs, d)
    nb, hkv, T = 211, 4, 1500
    x = W.chunk_elems(dtype)
    kc, vc = _random_cache((nb, hkv, d // x, bs, x), (nb, hkv, d, bs), dtype, 11)
    rng = np.random.default_rng(12)
    pages = rng.permutation(nb)
    slots = np.full(T, -1, dtype=np.int64)
    pos, p = 0, 0
    for run in (5, 300, 77, 640, 129):                  # prefill runs, each from a page offset onward
        start = int(rng.integers(0, bs))
        taken = []
        while len(taken) < run:
            taken.extend(int(pages[p]) * bs + o for o in range(start, bs))
            start, p = 0, p + 1
        slots[pos:pos + run] = taken[:run]
        pos += run + 3                                  # three padding tokens between runs
    free = np.array([int(q) * bs + o for q in pages[p:] for o in range(bs)], dtype=np.int64)
    slots[pos:] = rng.choice(free, size=T - pos, replace=False)     # scattered tail
    slots[[10, 400, 1490]] = [nb * bs, nb * bs + 99, -5]            # out of range / padding: skipped
    assert len(set(slots[slots >= 0].tolist())) == int((slots >= 0).sum())
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    td = W.torch_dtype(dtype)
    k = torch.randn(T, hkv, d, generator=g, device="cuda").to(td)
    v = torch.randn(T, hkv, d, generator=g, device="cuda").to(td)
    k_before, v_before = storage_np(kc), storage_np(vc)
    pa.kv_append(k, v, torch.from_numpy(slots).cuda(), kc, vc)
    torch.cuda.synchronize()
    ref_slots = np.where(slots >= nb * bs, -1, slots)
    rk, rv = oracle.kv_append(storage_np(k), storage_np(v), ref_slots, k_before, v_before, bs)
    view = np.uint16 if dtype == "bf16" else np.uint32
    assert np.array_equal(storage_np(kc).view(view), rk.view(view))
    assert np.array_equal(storage_np(vc).view(view), rv.view(view))


@pytest.mark.parametrize("dtype,bs,d", SHAPES)
def test_copy_blocks_bit_exact(dtype, bs, d):
    pa = require_gpu()
    say("copy_blocks", dtype, bs, d)
    nb, hkv = 41, 8
    x = W.chunk_elems(dtype)
    kc, vc = _random_cache((nb, hkv, d // x, bs, x), (nb, hkv, d, bs), dtype, 4)
    rng = np.random.default_rng(5)
    ids = rng.permutation(nb)
    pairs = np.stack([ids[:12], ids[12:24]], axis=1).astype(np.int64)
    pairs = np.concatenate([pairs, [[nb + 3, ids[30]], [ids[31], -2]]])   # skipped by the guard
    k_before, v_before = storage_np(kc), storage_np(vc)
    pa.copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    rk, rv = oracle.copy_blocks(k_before, v_before, pairs[:12])
    view = np.uint16 if dtype == "bf16" else np.uint32
    assert np.array_equal(storage_np(kc).view(view), rk.view(view))
    assert np.array_equal(storage_np(vc).view(view), rv.view(view))


def test_empty_calls_are_no_ops():
    pa = require_gpu()
    say("empty append/copy")
    kc, vc = _random_cache((4, 2, 16, 16, 8), (4, 2, 128, 16), "bf16", 6)
    k0, v0 = kc.clone(), vc.clone()
    e = torch.empty(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    pa.kv_append(e, e, torch.empty(0, dtype=torch.int64, device="cuda"), kc, vc)
    pa.copy_blocks(kc, vc, torch.empty(0, 2, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert bits_equal(kc, k0) and bits_equal(vc, v0)


def check_step_updates(pa, w, t):
    """Run the step's copies + appends and check them bit-exactly: touched
    pages against the oracle, every other page unchanged."""
    bs = w.block_size
    kc0, vc0 = t["k_cache"].clone(), t["v_cache"].clone()
    run_step_updates(pa, w, t)
    torch.cuda.synchronize()
    dst = set(w.copy_pairs[:, 1].tolist())
    touched = dst | set((w.append_slots // bs).tolist())
    pages = sorted(touched | set(w.copy_pairs[:, 0].tolist()))
    keep = torch.ones(w.num_blocks, dtype=torch.bool, device="cuda")
    keep[torch.tensor(sorted(touched), dtype=torch.long, device="cuda")] = False
    assert bits_equal(t["k_cache"][keep], kc0[keep]), "untouched K pages changed"
    assert bits_equal(t["v_cache"][keep], vc0[keep]), "untouched V pages changed"
    where = {p: i for i, p in enumerate(pages)}
    idx = torch.tensor(pages, dtype=torch.long, device="cuda")
    sub_k0, sub_v0 = storage_np(kc0.index_select(0, idx)), storage_np(vc0.index_select(0, idx))
    pairs = np.array([[where[int(s)], where[int(d)]] for s, d in w.copy_pairs], np.int64).reshape(-1, 2)
    slots = np.array([where[int(s) // bs] * bs + int(s) % bs for s in w.append_slots], np.int64)
    rk, rv = oracle.copy_blocks(sub_k0, sub_v0, pairs)
    rk, rv = oracle.kv_append(storage_np(t["k_new"]), storage_np(t["v_new"]), slots, rk, rv, bs)
    got_k = storage_np(t["k_cache"].index_select(0, idx))
    got_v = storage_np(t["v_cache"].index_select(0, idx))
    view = np.uint16 if w.dtype == "bf16" else np.uint32
    assert np.array_equal(got_k.view(view), rk.view(view)), "K pages differ from the oracle"
    assert np.array_equal(got_v.view(view), rv.view(view)), "V pages differ from the oracle"


@pytest.mark.parametrize("name", ["tiny", "llama3_8b", "prefix_share", "beam_fork", "long_context",
                                  "llama3_70b"])
def test_workload_step_updates_bit_exact(name):
    pa = require_gpu()
    w = W.by_name(name)
    say("step updates", name, w.summary())
    t = W.make_tensors(w, "cuda")
    check_step_updates(pa, w, t)


@pytest.mark.parametrize("scatter", [False, True])
def test_copy_probe_throughput_shape(scatter):
    """The eager-fork probe the benchmark times (7 x 1024 pages of 32 tokens,
    8 kv heads, D 128, bf16) against the oracle's copy, whole pool compared
    bit for bit: every destination page equals its source as it was, and
    every other page -- the sources and 512 spare pages -- is unchanged.
    With ``scatter`` the probe's page ids are sent through a seeded
    permutation of the larger pool, so copied and untouched pages
    interleave."""
    pa = require_gpu()
    pairs = W.copy_probe()
    nb = int(pairs.max()) + 1 + 512
    if scatter:
        perm = np.random.default_rng(8).permutation(nb).astype(np.int64)
        pairs = perm[pairs]
    say("copy probe", pairs.shape, nb, "scatter" if scatter else "as timed")
    kc, vc = _random_cache((nb, 8, 16, 32, 8), (nb, 8, 128, 32), "bf16", 7)
    k_before, v_before = storage_np(kc), storage_np(vc)
    rk, rv = oracle.copy_blocks(k_before, v_before, pairs)
    del k_before, v_before
    pa.copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(storage_np(kc), rk), "K pool differs from the oracle's copy"
    assert np.array_equal(storage_np(vc), rv), "V pool differs from the oracle's copy"
