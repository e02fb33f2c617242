"""Randomised shapes on the GPU against the float64 oracle.

The fixed-shape tests pin each path on purpose, one parameter at a time.
This sweep crosses the parameters with each other: every seed draws one
configuration -- block size, head dim, kv heads, query heads per kv head (1
to 16), batch size, ragged context lengths from 1 token to a few thousand,
partition sizes and load path -- and checks on it

* pa_decode, both kernels where the dtype has them, every drawn partition
  size and both load paths;
* pa_decode_append: caches bit-identical to the oracle's append, the output
  bit-identical to pa_kv_append + pa_decode and within tolerance of the
  oracle;
* pa_decode_multi with a random number of new tokens per sequence;
* pa_decode_shared_prefix over a random shared length, and
  pa_decode_shared_prefix_groups over random groups (sizes, shared lengths,
  groups that share nothing, a sequence in no group), plain and with the
  fused append;
* pa_kv_append of a random slot pattern (prefill runs starting anywhere in
  a page, scattered slots, padding, slots outside the pool), bit-exact on
  the whole cache.

Seeds are fixed, so every run checks the same cases."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bits_equal, check_close, out_f64, require_gpu, say, step_and_reference, storage_np
from test_gpu_cache_ops import _random_cache
from test_gpu_fused import newest_rows
from test_gpu_multi import oracle_multi, prepare
from test_gpu_shared_prefix import _grouped_batch

pytestmark = pytest.mark.gpu

SEEDS = list(range(30))
GROUPS = [1, 2, 3, 4, 5, 6, 7, 8, 12, 16]
PARTS = [-1, 0, 32, 64, 96, 160, 512, 2048]


def _draw(seed):
    """One configuration: (rng, block_size, head_dim, kv heads, group,
    context lengths, three partition sizes)."""
    rng = np.random.default_rng(9100 + seed)
    bs = int(rng.choice([16, 32]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice(GROUPS))
    nseq = int(rng.integers(1, 25))
    longer = rng.random(nseq) < 0.7
    lens = np.where(longer, rng.integers(1, 2500, size=nseq, endpoint=True),
                    rng.integers(1, 70, size=nseq, endpoint=True))
    parts = [int(x) for x in rng.choice(PARTS, size=3, replace=False)]
    return rng, bs, d, hkv, g, lens, parts


def _decode(pa, w, t, P, kernel, reuse):
    return pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"], w.scale,
                     w.max_context_len, partition_size=P, kernel=kernel, reuse=reuse)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_decode(seed):
    pa = require_gpu()
    rng, bs, d, hkv, g, lens, parts = _draw(seed)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    w = W.custom(f"random_decode_{seed}", 9100 + seed, dtype, lens.tolist(), g * hkv, hkv, d, bs)
    say("random decode seed", seed, "partitions", parts, w.summary())
    t = W.make_tensors(w, "cuda")
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    for kernel in (["valu", "mfma"] if dtype == "bf16" else ["valu"]):
        for reuse in ("stream", "shared"):
            for P in parts:
                say("  kernel", kernel, "reuse", reuse, "partition", P)
                out = _decode(pa, w, t, P, kernel, reuse)
                torch.cuda.synchronize()
                check_close(out_f64(out), ref, dtype, f"seed {seed} {kernel} {reuse} P={P}")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_fused_append(seed):
    pa = require_gpu()
    rng, bs, d, hkv, g, lens, parts = _draw(seed)
    w = W.custom(f"random_fused_{seed}", 9100 + seed, "bf16", lens.tolist(), g * hkv, hkv, d, bs)
    say("random fused append seed", seed, "partitions", parts, w.summary())
    t = W.make_tensors(w, "cuda")
    k_new, v_new, mask, older = newest_rows(w, t)
    assert not older
    kc0, vc0 = storage_np(t["k_cache"]), storage_np(t["v_cache"])
    kc_ref, vc_ref = oracle.kv_append(storage_np(k_new)[mask >= 0], storage_np(v_new)[mask >= 0], mask[mask >= 0],
                                      kc0, vc0, bs)
    ref = oracle.decode(storage_np(t["q"]), kc_ref, vc_ref, w.block_tables, w.context_lens, w.scale, bs, "bf16")
    mask_t = torch.from_numpy(mask).cuda()
    for reuse in ("stream", "shared"):
        for P in parts:
            say("  reuse", reuse, "partition", P)
            fused = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
            out = pa.decode_append(k_new, v_new, fused["q"], fused["k_cache"], fused["v_cache"],
                                   fused["block_tables"], fused["context_lens"], w.scale, w.max_context_len,
                                   slot_mapping=mask_t, partition_size=P, reuse=reuse)
            apart = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
            pa.kv_append(k_new[mask_t >= 0].contiguous(), v_new[mask_t >= 0].contiguous(),
                         mask_t[mask_t >= 0].contiguous(), apart["k_cache"], apart["v_cache"])
            two = _decode(pa, w, apart, P, "auto", reuse)
            torch.cuda.synchronize()
            assert np.array_equal(storage_np(fused["k_cache"]), kc_ref), f"seed {seed} K cache P={P}"
            assert np.array_equal(storage_np(fused["v_cache"]), vc_ref), f"seed {seed} V cache P={P}"
            assert bits_equal(out, two), f"seed {seed} fused vs separate {reuse} P={P}"
            check_close(out_f64(out), ref, "bf16", f"seed {seed} fused {reuse} P={P}")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_multi_query(seed):
    pa = require_gpu()
    rng, bs, d, hkv, g, lens, parts = _draw(seed)
    news = np.minimum(lens, rng.integers(0, 13, size=len(lens)))
    w = W.multi_custom(f"random_multi_{seed}", 9100 + seed, lens.tolist(), news.tolist(), g * hkv, hkv, d, bs)
    t, kc0, vc0, q = prepare(w)
    say("random multi-query seed", seed, "new tokens", news.tolist(), "partitions", parts, w.summary())
    ref = oracle_multi(w, kc0, vc0, q)
    pa.kv_append(t["k_new"], t["v_new"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    for reuse in ("stream", "shared"):
        for P in parts:
            say("  reuse", reuse, "partition", P)
            out = pa.decode_multi(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  t["query_start"], w.scale, w.max_context_len, w.max_query_len,
                                  partition_size=P, reuse=reuse)
            torch.cuda.synchronize()
            check_close(out_f64(out), ref, "bf16", f"seed {seed} multi {reuse} P={P}")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shared_prefix(seed):
    """Every sequence reads row 0's pages for its first S positions; each
    context goes at least one token past them (the appended row never lands
    in a shared page)."""
    pa = require_gpu()
    rng, bs, d, hkv, g, _, parts = _draw(seed)
    nseq = int(rng.integers(1, 41))
    shared = bs * int(rng.integers(1, 2000 // bs))
    lens = shared + 1 + rng.integers(0, 600, size=nseq)
    w = W.custom(f"random_shared_{seed}", 9100 + seed, "bf16", lens.tolist(), g * hkv, hkv, d, bs)
    t = W.make_tensors(w, "cuda")
    tables = w.block_tables.copy()
    tables[:, :shared // bs] = tables[0, :shared // bs]
    w.block_tables = tables
    t["block_tables"].copy_(torch.from_numpy(tables))
    say("random shared prefix seed", seed, "shared", shared, "partitions", parts, w.summary())
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    assert pa.shared_prefix_len(w.block_tables, w.context_lens, bs) >= shared
    for P in [0] + [p for p in parts if p > 0]:
        say("  partition", P)
        out = pa.decode_shared_prefix(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                      w.scale, w.max_context_len, shared, P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"seed {seed} shared prefix P={P}")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_prefix_groups(seed):
    pa = require_gpu()
    rng, bs, d, hkv, g, _, parts = _draw(seed)
    groups = [(int(rng.integers(1, 31)), 0 if rng.random() < 0.2 else bs * int(rng.integers(1, 1500 // bs)))
              for _ in range(int(rng.integers(1, 7)))]
    w, t, arr = _grouped_batch(9700 + seed, g * hkv, hkv, d, bs, groups, loner_len=int(rng.integers(1, 900)))
    say("random prefix groups seed", seed, groups, "partitions", parts, w.summary())
    fused = rng.random() < 0.5
    if not fused:
        ref = step_and_reference(pa, w, t, range(w.num_seqs))
        for P in [0] + [p for p in parts if p > 0]:
            say("  partition", P)
            out = pa.decode_shared_prefix_groups(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                                 t["context_lens"], w.scale, w.max_context_len, partition_size=P,
                                                 **arr)
            torch.cuda.synchronize()
            check_close(out_f64(out), ref, "bf16", f"seed {seed} groups P={P}")
        return
    k_new, v_new, mask, older = newest_rows(w, t)
    assert not older
    kc0, vc0 = storage_np(t["k_cache"]), storage_np(t["v_cache"])
    rk, rv = oracle.kv_append(storage_np(k_new), storage_np(v_new), mask, kc0, vc0, bs)
    ref = oracle.decode(storage_np(t["q"]), rk, rv, w.block_tables, w.context_lens, w.scale, bs, "bf16")
    for P in [0] + [p for p in parts if p > 0]:
        say("  fused append, partition", P)
        kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
        out = pa.decode_shared_prefix_groups(t["q"], kc, vc, t["block_tables"], t["context_lens"], w.scale,
                                             w.max_context_len, partition_size=P, k_new=k_new, v_new=v_new,
                                             slot_mapping=torch.from_numpy(mask).cuda(), **arr)
        torch.cuda.synchronize()
        assert np.array_equal(storage_np(kc).view(np.uint16), rk.view(np.uint16)), f"seed {seed} K cache P={P}"
        assert np.array_equal(storage_np(vc).view(np.uint16), rv.view(np.uint16)), f"seed {seed} V cache P={P}"
        check_close(out_f64(out), ref, "bf16", f"seed {seed} groups fused P={P}")

def append_slots(rng, T, bs):
    """A slot pattern of T tokens and the pool it needs: prefill runs
    (positions a .. a + n - 1 of a sequence whose pages come off a permuted
    free list, so a run may start anywhere in its first page), single
    scattered slots, padding (-1) and slots past the pool.  Every valid slot
    is unique: each page serves one run or one scattered slot."""
    nb = 3 * (T // bs) + 200
    free = [int(x) for x in rng.permutation(nb)]
    slots = []
    while len(slots) < T:
        kind = rng.random()
        if kind < 0.6:
            a = int(rng.integers(0, 3 * bs))
            n = int(rng.integers(1, 300))
            need = (a + n + bs - 1) // bs
            if need > len(free):
                slots.append(-1)
                continue
            pages = [free.pop() for _ in range(need)]
            slots.extend(pages[p // bs] * bs + p % bs for p in range(a, a + n))
        elif kind < 0.8 and free:
            slots.append(free.pop() * bs + int(rng.integers(0, bs)))
        elif kind < 0.9:
            slots.append(-1)
        else:
            slots.append(nb * bs + int(rng.integers(0, 1000)))
    return np.asarray(slots[:T], dtype=np.int64), nb


@pytest.mark.parametrize("seed", SEEDS)
def test_random_append(seed):
    pa = require_gpu()
    rng = np.random.default_rng(9400 + seed)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    bs = int(rng.choice([16, 32]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    T = int(rng.integers(1, 512)) if rng.random() < 0.4 else int(rng.integers(512, 6000))
    slots, nb = append_slots(rng, T, bs)
    say("random append seed", seed, dtype, "bs", bs, "D", d, "kv heads", hkv, "tokens", T, "pages", nb)
    x = W.chunk_elems(dtype)
    kc, vc = _random_cache((nb, hkv, d // x, bs, x), (nb, hkv, d, bs), dtype, 9400 + seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(9400 + seed)
    td = W.torch_dtype(dtype)
    k = torch.randn(T, hkv, d, generator=g, device="cuda").to(td)
    v = torch.randn(T, hkv, d, generator=g, device="cuda").to(td)
    k_before, v_before = storage_np(kc), storage_np(vc)
    pa.kv_append(k, v, torch.from_numpy(slots).cuda(), kc, vc)
    torch.cuda.synchronize()
    ref_slots = np.where(slots < nb * bs, slots, -1)         # slots past the pool write nothing
    rk, rv = oracle.kv_append(storage_np(k), storage_np(v), ref_slots, k_before, v_before, bs)
    view = np.uint16 if dtype == "bf16" else np.uint32
    assert np.array_equal(storage_np(kc).view(view), rk.view(view)), f"seed {seed} K cache"
    assert np.array_equal(storage_np(vc).view(view), rv.view(view)), f"seed {seed} V cache"
