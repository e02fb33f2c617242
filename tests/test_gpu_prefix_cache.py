"""Decode over pages shared by prompt content (prefix caching), on the GPU.

Requests over two system prompts (and some with none) are admitted through
the native manager's allocate_prompt: K/V rows are written (pa_kv_append)
only for the tokens after each request's cached prefix, some requests are
freed and new ones admitted (so cached pages are taken back off the free
list and others evicted), and each live request then gets one decode step
through pa_decode_append.  The check: every output equals the oracle decode
of the same logical K/V rows laid out privately, page by page, in a host
cache of its own -- so a shared page must hold exactly the rows each of its
holders would have written."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import check_close, out_f64, require_gpu, say, storage_np

pytestmark = pytest.mark.gpu


BS, HQ, HKV, D, NB = 16, 32, 8, 128, 600


def plan(pa):
    """Host half (no device calls): the manager's decisions and the rows.
    Returns the manager, the row writes in issue order, the live requests'
    logical rows, and counts of cache hits and of pages taken back off the
    free list."""
    rng = np.random.default_rng(41)
    g = torch.Generator(device="cpu")
    g.manual_seed(42)

    def rows(n):
        return (torch.randn(n, HKV, D, generator=g).to(torch.bfloat16),
                torch.randn(n, HKV, D, generator=g).to(torch.bfloat16))

    # the "model": a system prompt's tokens have the same K/V in every
    # request that starts with it; the rest of a request's rows are its own
    systems = []
    for n in (100, 333):
        k, v = rows(n)
        systems.append((rng.integers(0, 128256, size=n).tolist(), k, v))
    m = pa.NativeBlockManager(NB, BS, free_order=rng.permutation(NB))
    writes = []                      # (slots, K rows, V rows) in issue order
    logical = {}                     # live seq -> (K rows, V rows) of all its tokens
    spec = {}                        # every admitted seq -> (tokens, K rows, V rows)

    def write(seq, toks, k_all, v_all):
        spec[seq] = (toks, k_all, v_all)
        free_before = set(m.free_list())
        pages, cached = m.allocate_prompt(seq, toks)
        if cached < len(toks):
            pos = np.arange(cached, len(toks))
            slots = np.array(pages, dtype=np.int64)[pos // BS] * BS + pos % BS
            writes.append((slots, k_all[cached:], v_all[cached:]))
        logical[seq] = (k_all, v_all)
        return cached, len(free_before & set(pages[:cached // BS]))

    def admit(seq):
        sysid = int(rng.integers(0, 3))
        if sysid < 2:
            toks, sk, sv = systems[sysid]
            cut = int(rng.integers(len(toks) // 2, len(toks) + 1))
            toks, sk, sv = toks[:cut], sk[:cut], sv[:cut]
        else:
            toks = []
            sk = sv = torch.empty(0, HKV, D, dtype=torch.bfloat16)
        extra = int(rng.integers(0, 40))
        ek, ev = rows(extra)
        toks = toks + rng.integers(0, 128256, size=extra).tolist()
        return write(seq, toks, torch.cat([sk, ek]), torch.cat([sv, ev]))

    hits = revived = 0
    for s in range(10):
        hits += admit(s)[0] > 0
    for s in (1, 4, 7):                          # pages only they held go back to the free list
        m.free_sequence(s)
        del logical[s]
    for s in range(10, 16):
        hits += admit(s)[0] > 0
    for s, old in ((16, 1), (17, 4), (18, 7)):   # the freed prompts again
        toks = spec[old][0]
        cached, back = write(s, *spec[old])
        assert cached == len(toks) // BS * BS    # every full page is still cached
        revived += back
    return m, writes, logical, hits, revived, rows, g


def test_decode_over_prefix_cached_pages():
    pa = require_gpu()
    m, writes, logical, hits, revived, rows, g = plan(pa)
    assert hits >= 4 and revived >= 1
    say("cached pages", m.num_cached(), "free", m.num_free(), "hits", hits, "taken back", revived)
    x = W.chunk_elems("bf16")
    scale = float(np.float32(1.0 / np.sqrt(D)))
    nan = float("nan")
    kc = torch.full((NB, HKV, D // x, BS, x), nan, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((NB, HKV, D, BS), nan, dtype=torch.bfloat16, device="cuda")
    for slots, k, v in writes:
        pa.kv_append(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), kc, vc)

    live = sorted(logical)
    ids = np.array(live, dtype=np.int64)
    maxb = max(len(m.pages(s)) for s in live) + 2
    tables, lens = m.block_tables(ids, maxb, pad_page=NB - 1)
    tables, lens = tables.copy(), lens.copy()
    slots, copies = m.append(ids, tables, lens)
    assert len(copies) == 0                       # a partly filled page is never shared by content
    k_new, v_new = rows(len(live))
    q = torch.randn(len(live), HQ, D, generator=g).to(torch.bfloat16)
    out = pa.decode_append(k_new.cuda(), v_new.cuda(), q.cuda(), kc, vc, torch.from_numpy(tables).cuda(),
                           torch.from_numpy(lens).cuda(), scale, int(lens.max()),
                           slot_mapping=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()

    # oracle: the same logical rows in a private layout of their own
    L = [int(logical[s][0].shape[0]) + 1 for s in live]     # every row written, plus the new one
    assert lens.tolist() == L
    npages = [-(-n // BS) for n in L]
    pk = np.zeros((sum(npages) + 1, HKV, D // x, BS, x), dtype=np.uint16)
    pv = np.zeros((sum(npages) + 1, HKV, D, BS), dtype=np.uint16)
    ptab = np.zeros((len(live), max(npages)), dtype=np.int32)
    base = 0
    for i, s in enumerate(live):
        ptab[i, :npages[i]] = np.arange(base, base + npages[i])
        k_all = torch.cat([logical[s][0], k_new[i:i + 1]])
        v_all = torch.cat([logical[s][1], v_new[i:i + 1]])
        slot = np.arange(L[i], dtype=np.int64) + base * BS
        pk, pv = oracle.kv_append(storage_np(k_all), storage_np(v_all), slot, pk, pv, BS)
        base += npages[i]
    ref = oracle.decode(storage_np(q), pk, pv, ptab, np.array(L, dtype=np.int32), scale, BS, "bf16")
    check_close(out_f64(out), ref, "bf16", "prefix-cached decode")
