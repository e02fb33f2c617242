"""Decode steps driven end to end by the native page allocator, on the GPU.

Six sequences fork one 40-token prompt (its last page is shared and partly
filled, so their first appends copy-on-write) and four more run on their own.
Every step the manager appends a token to each sequence and keeps the block
tables current in place; its copy pairs go to pa_copy_blocks, the new rows to
pa_decode_append (or pa_kv_append + pa_decode on alternate steps).

The oracle's page pool runs the same calls in lockstep: the manager's slots
and copy pairs must equal the pool's, and the oracle decode takes the pool's
own block tables and lengths.  A host mirror of the caches is updated with
the oracle's copy and append; each step's output is checked against the
oracle decode and the caches bit for bit at the end."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import check_close, out_f64, require_gpu, say, storage_np

pytestmark = pytest.mark.gpu


def test_decode_loop_driven_by_native_manager():
    pa = require_gpu()
    bs, hq, hkv, d, nb, maxb, steps = 16, 32, 8, 128, 300, 10, 14
    rng = np.random.default_rng(31)
    order = rng.permutation(nb)
    m = pa.NativeBlockManager(nb, bs, free_order=order)
    pool = oracle.PrefixCachingPool(nb, bs, free_order=order.tolist())
    g = torch.Generator(device="cuda")
    g.manual_seed(32)

    def rows(n):
        return (torch.randn(n, hkv, d, generator=g, device="cuda").to(torch.bfloat16),
                torch.randn(n, hkv, d, generator=g, device="cuda").to(torch.bfloat16))

    x = W.chunk_elems("bf16")
    nan = float("nan")
    kc = torch.full((nb, hkv, d // x, bs, x), nan, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((nb, hkv, d, bs), nan, dtype=torch.bfloat16, device="cuda")
    hk, hv = storage_np(kc), storage_np(vc)                 # host mirror

    def pool_tables(ids):
        t = np.full((len(ids), maxb), nb - 1, dtype=np.int32)
        for i, b in enumerate(ids):
            t[i, :len(pool.pages[b])] = pool.pages[b]
        return t, np.array([pool.length[b] for b in ids], dtype=np.int32)

    def prefill(seq, n):
        slots, copies = m.append(np.full(n, seq, dtype=np.int64))
        assert len(copies) == 0
        pslots = [pool.append_token(seq) for _ in range(n)]
        assert slots.tolist() == pslots
        k, v = rows(n)
        pa.kv_append(k, v, torch.from_numpy(slots).cuda(), kc, vc)
        return oracle.kv_append(storage_np(k), storage_np(v), pslots, hk, hv, bs)

    m.allocate(0, 0)
    pool.allocate(0, 0)
    hk, hv = prefill(0, 40)
    for child in range(1, 6):
        m.fork(0, child)
        pool.fork(0, child)
    for s in range(6, 10):
        m.allocate(s, 0)
        pool.allocate(s, 0)
        hk, hv = prefill(s, int(rng.integers(1, 100)))
    ids = np.arange(10, dtype=np.int64)
    tables, lens = m.block_tables(ids, maxb, pad_page=nb - 1)
    tables, lens = tables.copy(), lens.copy()
    scale = float(np.float32(1.0 / np.sqrt(d)))
    copies_seen = 0
    for step in range(steps):
        slots, copies = m.append(ids, tables, lens)
        copies_seen += len(copies)
        before = len(pool.copies)
        pslots = [pool.append_token(int(b)) for b in ids]
        assert slots.tolist() == pslots
        assert [tuple(c) for c in np.asarray(copies).reshape(-1, 2).tolist()] == pool.copies[before:]
        ptables, plens = pool_tables(ids.tolist())
        assert np.array_equal(ptables, tables) and np.array_equal(plens, lens)
        say("step", step, "copies", copies.tolist())
        if len(copies):
            pa.copy_blocks(kc, vc, torch.from_numpy(np.ascontiguousarray(copies)).cuda())
            hk, hv = oracle.copy_blocks(hk, hv, np.array(pool.copies[before:], dtype=np.int64))
        k, v = rows(len(ids))
        q = torch.randn(len(ids), hq, d, generator=g, device="cuda").to(torch.bfloat16)
        bt = torch.from_numpy(tables).cuda()
        cl = torch.from_numpy(lens).cuda()
        maxctx = int(lens.max())
        if step % 2 == 0:
            out = pa.decode_append(k, v, q, kc, vc, bt, cl, scale, maxctx,
                                   slot_mapping=torch.from_numpy(slots).cuda(), reuse="shared")
        else:
            pa.kv_append(k, v, torch.from_numpy(slots).cuda(), kc, vc)
            out = pa.decode(q, kc, vc, bt, cl, scale, maxctx, reuse="shared")
        torch.cuda.synchronize()
        hk, hv = oracle.kv_append(storage_np(k), storage_np(v), pslots, hk, hv, bs)
        ref = oracle.decode(storage_np(q), hk, hv, ptables, plens, scale, bs, "bf16")
        check_close(out_f64(out), ref, "bf16", f"step {step}")
    assert copies_seen == 5                                  # five children leave the shared page
    assert np.array_equal(storage_np(kc).view(np.uint16), hk.view(np.uint16))
    assert np.array_equal(storage_np(vc).view(np.uint16), hv.view(np.uint16))


def test_beams_driven_by_native_manager_through_the_shared_prefix_path():
    """Eight beams fork one 200-token prompt (its last page partly filled).
    Every step the manager appends a token to each beam (the first step copies
    the shared tail page for each of them), its copy pairs go to
    pa_copy_blocks, and pa_decode_shared_prefix appends the rows and decodes,
    with the shared length the manager reports.  The oracle's pool runs in
    lockstep; each step's output is checked against the oracle decode and the
    caches bit for bit at the end."""
    pa = require_gpu()
    bs, hq, hkv, d, nb, maxb, steps = 16, 32, 8, 128, 200, 16, 6
    rng = np.random.default_rng(41)
    order = rng.permutation(nb)
    m = pa.NativeBlockManager(nb, bs, free_order=order)
    pool = oracle.PrefixCachingPool(nb, bs, free_order=order.tolist())
    g = torch.Generator(device="cuda")
    g.manual_seed(42)

    def rows(n):
        return (torch.randn(n, hkv, d, generator=g, device="cuda").to(torch.bfloat16),
                torch.randn(n, hkv, d, generator=g, device="cuda").to(torch.bfloat16))

    x = W.chunk_elems("bf16")
    nan = float("nan")
    kc = torch.full((nb, hkv, d // x, bs, x), nan, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((nb, hkv, d, bs), nan, dtype=torch.bfloat16, device="cuda")
    hk, hv = storage_np(kc), storage_np(vc)

    m.allocate(0, 0)
    pool.allocate(0, 0)
    slots0, _ = m.append(np.full(200, 0, dtype=np.int64))
    pslots0 = [pool.append_token(0) for _ in range(200)]
    assert slots0.tolist() == pslots0
    k0, v0 = rows(200)
    pa.kv_append(k0, v0, torch.from_numpy(slots0).cuda(), kc, vc)
    hk, hv = oracle.kv_append(storage_np(k0), storage_np(v0), pslots0, hk, hv, bs)
    beams = np.arange(1, 9, dtype=np.int64)
    for b in beams.tolist():
        m.fork(0, b)
        pool.fork(0, b)
    tables, lens = m.block_tables(beams, maxb, pad_page=nb - 1)
    tables, lens = tables.copy(), lens.copy()
    scale = float(np.float32(1.0 / np.sqrt(d)))
    for step in range(steps):
        slots, copies = m.append(beams, tables, lens)
        before = len(pool.copies)
        pslots = [pool.append_token(int(b)) for b in beams]
        assert slots.tolist() == pslots
        shared = m.shared_prefix(beams)
        assert shared == 192                                  # the prompt's 12 whole pages
        say("beam step", step, "copies", len(copies), "shared_len", shared)
        if len(copies):
            pa.copy_blocks(kc, vc, torch.from_numpy(np.ascontiguousarray(copies)).cuda())
            hk, hv = oracle.copy_blocks(hk, hv, np.array(pool.copies[before:], dtype=np.int64))
        k, v = rows(len(beams))
        q = torch.randn(len(beams), hq, d, generator=g, device="cuda").to(torch.bfloat16)
        out = pa.decode_shared_prefix(q, kc, vc, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                                      scale, int(lens.max()), shared, 64, k_new=k, v_new=v,
                                      slot_mapping=torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        hk, hv = oracle.kv_append(storage_np(k), storage_np(v), pslots, hk, hv, bs)
        ptables = np.full((len(beams), maxb), nb - 1, dtype=np.int32)
        for i, b in enumerate(beams.tolist()):
            ptables[i, :len(pool.pages[b])] = pool.pages[b]
        plens = np.array([pool.length[b] for b in beams.tolist()], dtype=np.int32)
        assert np.array_equal(ptables, tables) and np.array_equal(plens, lens)
        ref = oracle.decode(storage_np(q), hk, hv, ptables, plens, scale, bs, "bf16")
        check_close(out_f64(out), ref, "bf16", f"beam step {step}")
    assert np.array_equal(storage_np(kc).view(np.uint16), hk.view(np.uint16))
    assert np.array_equal(storage_np(vc).view(np.uint16), hv.view(np.uint16))


def test_prompt_groups_driven_by_native_manager():
    """Two prompts (150 and 96 tokens) forked to 5 and 4 sequences, with a
    sequence on its own between them.  Every step the manager appends a token
    to each, its copy pairs go to pa_copy_blocks, and
    pa_decode_shared_prefix_groups appends the rows and decodes with the group
    arrays the manager reports (pa_bm_prefix_groups).  The oracle's pool runs
    in lockstep; outputs against the oracle decode every step, caches bit for
    bit at the end."""
    pa = require_gpu()
    bs, hq, hkv, d, nb, maxb, steps = 16, 32, 8, 128, 240, 16, 5
    rng = np.random.default_rng(51)
    order = rng.permutation(nb)
    m = pa.NativeBlockManager(nb, bs, free_order=order)
    pool = oracle.PrefixCachingPool(nb, bs, free_order=order.tolist())
    g = torch.Generator(device="cuda")
    g.manual_seed(52)

    def rows(n):
        return (torch.randn(n, hkv, d, generator=g, device="cuda").to(torch.bfloat16),
                torch.randn(n, hkv, d, generator=g, device="cuda").to(torch.bfloat16))

    x = W.chunk_elems("bf16")
    nan = float("nan")
    kc = torch.full((nb, hkv, d // x, bs, x), nan, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((nb, hkv, d, bs), nan, dtype=torch.bfloat16, device="cuda")
    hk, hv = storage_np(kc), storage_np(vc)

    def prefill(seq, n):
        nonlocal hk, hv
        m.allocate(seq, 0)
        pool.allocate(seq, 0)
        slots, _ = m.append(np.full(n, seq, dtype=np.int64))
        pslots = [pool.append_token(seq) for _ in range(n)]
        assert slots.tolist() == pslots
        k, v = rows(n)
        pa.kv_append(k, v, torch.from_numpy(slots).cuda(), kc, vc)
        hk, hv = oracle.kv_append(storage_np(k), storage_np(v), pslots, hk, hv, bs)

    prefill(100, 150)
    prefill(200, 96)
    for c in (1, 2, 3, 4, 5):
        m.fork(100, c)
        pool.fork(100, c)
    prefill(6, 70)
    for c in (7, 8, 9, 10):
        m.fork(200, c)
        pool.fork(200, c)
    batch = np.array([1, 2, 3, 4, 5, 6, 7, 8, 9, 10], dtype=np.int64)
    tables, lens = m.block_tables(batch, maxb, pad_page=nb - 1)
    tables, lens = tables.copy(), lens.copy()
    scale = float(np.float32(1.0 / np.sqrt(d)))
    for step in range(steps):
        slots, copies = m.append(batch, tables, lens)
        before = len(pool.copies)
        pslots = [pool.append_token(int(b)) for b in batch]
        assert slots.tolist() == pslots
        gs, gl, sl, max_group, max_shared = m.prefix_groups(batch)
        assert gs.tolist() == [0, 5, 6, 10] and gl.tolist() == [144, 0, 96]
        assert (max_group, max_shared) == (5, 144)
        say("groups step", step, "copies", len(copies))
        if len(copies):
            pa.copy_blocks(kc, vc, torch.from_numpy(np.ascontiguousarray(copies)).cuda())
            hk, hv = oracle.copy_blocks(hk, hv, np.array(pool.copies[before:], dtype=np.int64))
        k, v = rows(len(batch))
        q = torch.randn(len(batch), hq, d, generator=g, device="cuda").to(torch.bfloat16)
        out = pa.decode_shared_prefix_groups(
            q, kc, vc, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), scale, int(lens.max()),
            group_start=torch.from_numpy(gs).cuda(), group_shared_len=torch.from_numpy(gl).cuda(),
            seq_shared_len=torch.from_numpy(sl).cuda(), max_group_size=max_group,
            max_shared_len=max_shared, partition_size=64, k_new=k, v_new=v,
            slot_mapping=torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        hk, hv = oracle.kv_append(storage_np(k), storage_np(v), pslots, hk, hv, bs)
        ptables = np.full((len(batch), maxb), nb - 1, dtype=np.int32)
        for i, b in enumerate(batch.tolist()):
            ptables[i, :len(pool.pages[b])] = pool.pages[b]
        plens = np.array([pool.length[b] for b in batch.tolist()], dtype=np.int32)
        assert np.array_equal(ptables, tables) and np.array_equal(plens, lens)
        ref = oracle.decode(storage_np(q), hk, hv, ptables, plens, scale, bs, "bf16")
        check_close(out_f64(out), ref, "bf16", f"groups step {step}")
    assert np.array_equal(storage_np(kc).view(np.uint16), hk.view(np.uint16))
    assert np.array_equal(storage_np(vc).view(np.uint16), hv.view(np.uint16))
