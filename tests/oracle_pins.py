"""Checks that pin the oracle's attention to things other than itself.

Each ``pin_*`` takes the oracle module (so the mutation tests can hand in a
deliberately broken copy) and raises AssertionError on disagreement.  None of
them re-states the oracle's formula on the same data path:

* brute force   -- a pure-Python loop over a *contiguous* tensor, scattered
                   into a paged cache by an explicit per-element loop here;
* library       -- torch's scaled_dot_product_attention in float64 with its
                   own grouped-query convention (enable_gqa);
* closed forms  -- L = 1, zero scale, equal keys, a 3:1 two-token split, a
                   dominant key, identical query heads, L = 0;
* invariants    -- permuting physical pages (with the matching table edit),
                   padding the pool, poisoning unread slots.
"""

import math

import numpy as np
import torch

BS = 16


def contiguous_to_paged(K, V, table, block_size, num_blocks, x, fill=np.nan):
    """Scatter contiguous K/V [L, hkv, D] into paged caches, one element at a time.

    Layout: k_cache[page][h][d // x][off][d % x], v_cache[page][h][d][off].
    """
    L, hkv, d = K.shape
    kc = np.full((num_blocks, hkv, d // x, block_size, x), fill, dtype=np.float32)
    vc = np.full((num_blocks, hkv, d, block_size), fill, dtype=np.float32)
    for t in range(L):
        page = table[t // block_size]
        off = t % block_size
        for h in range(hkv):
            for e in range(d):
                kc[page, h, e // x, off, e % x] = K[t, h, e]
                vc[page, h, e, off] = V[t, h, e]
    return kc, vc


def brute_attention(q, K, V, scale, group):
    """Pure-Python softmax attention over contiguous lists (float64)."""
    hq, d = len(q), len(q[0])
    L = len(K)
    out = []
    for h in range(hq):
        g = h // group
        scores = []
        for t in range(L):
            acc = 0.0
            for e in range(d):
                acc += q[h][e] * K[t][g][e]
            scores.append(acc * scale)
        if L == 0:
            out.append([0.0] * d)
            continue
        top = max(scores)
        w = [math.exp(s - top) for s in scores]
        tot = sum(w)
        row = []
        for e in range(d):
            row.append(sum(w[t] * V[t][g][e] for t in range(L)) / tot)
        out.append(row)
    return out


def _f32(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _case(rng, L, hq, hkv, d, num_blocks, x=4, block_size=BS):
    K = _f32(rng, L, hkv, d)
    V = _f32(rng, L, hkv, d)
    q = _f32(rng, 1, hq, d)
    nblk = -(-L // block_size)
    table = [int(p) for p in rng.permutation(num_blocks)[:max(nblk, 1)]]
    kc, vc = contiguous_to_paged(K, V, table, block_size, num_blocks, x)
    return q, K, V, table, kc, vc


def pin_brute_force(oracle):
    rng = np.random.default_rng(11)
    for L, hq, hkv, d in [(1, 2, 1, 4), (17, 4, 2, 8), (36, 4, 4, 8), (40, 6, 3, 4), (32, 2, 2, 8)]:
        q, K, V, table, kc, vc = _case(rng, L, hq, hkv, d, num_blocks=8)
        scale = float(np.float32(0.37))
        tables = np.array([table + [table[0]] * 4], dtype=np.int32)
        got = oracle.decode(q, kc, vc, tables, np.array([L], np.int32), scale, BS, "f32")[0]
        want = np.array(brute_attention(q[0].astype(np.float64).tolist(),
                                        K.astype(np.float64).tolist(),
                                        V.astype(np.float64).tolist(), scale, hq // hkv))
        assert got.shape == want.shape
        assert np.allclose(got, want, rtol=0, atol=1e-12), (L, hq, hkv, d, np.abs(got - want).max())


def pin_library_sdpa(oracle):
    """torch SDPA (float64, CPU, enable_gqa) over the gathered sequence."""
    rng = np.random.default_rng(12)
    for L, hq, hkv, d, bs in [(36, 4, 4, 64, 16), (70, 8, 2, 16, 16), (95, 8, 1, 8, 32), (129, 12, 4, 16, 32)]:
        x = 4
        q, K, V, table, kc, vc = _case(rng, L, hq, hkv, d, num_blocks=12, x=x, block_size=bs)
        scale = float(np.float32(1 / math.sqrt(d)))
        tables = np.array([table], dtype=np.int32)
        got = oracle.decode(q, kc, vc, tables, np.array([L], np.int32), scale, bs, "f32")[0]
        tq = torch.from_numpy(q.astype(np.float64)).view(1, hq, 1, d)
        tk = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
        tv = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
        want = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, scale=scale, enable_gqa=True).view(hq, d).numpy()
        assert np.allclose(got, want, rtol=0, atol=1e-12), (L, hq, hkv, np.abs(got - want).max())


def _single(oracle, q, K, V, scale, block_size=BS, x=4, num_blocks=8, seed=0):
    rng = np.random.default_rng(seed)
    L = K.shape[0]
    table = [int(p) for p in rng.permutation(num_blocks)[:max(1, -(-L // block_size))]]
    kc, vc = contiguous_to_paged(K, V, table, block_size, num_blocks, x)
    return oracle.decode(q[None], kc, vc, np.array([table], np.int32),
                         np.array([L], np.int32), scale, block_size, "f32")[0]


def pin_closed_forms(oracle):
    rng = np.random.default_rng(13)
    hq, hkv, d = 4, 2, 8
    # L = 1: the only weight is 1, output = that value row exactly.
    K, V, q = _f32(rng, 1, hkv, d), _f32(rng, 1, hkv, d), _f32(rng, hq, d)
    out = _single(oracle, q, K, V, 0.5)
    for h in range(hq):
        assert np.array_equal(out[h], V[0, h // 2].astype(np.float64)), "L=1"
    # scale 0: uniform weights, output = mean of the value rows.
    K, V = _f32(rng, 23, hkv, d), _f32(rng, 23, hkv, d)
    out = _single(oracle, q, K, V, 0.0)
    for h in range(hq):
        assert np.allclose(out[h], V[:, h // 2].astype(np.float64).mean(0), atol=1e-14), "scale 0"
    # equal keys: uniform weights again, whatever the scale.
    Ke = np.repeat(_f32(rng, 1, hkv, d), 23, axis=0)
    out = _single(oracle, q, Ke, V, 0.9)
    for h in range(hq):
        assert np.allclose(out[h], V[:, h // 2].astype(np.float64).mean(0), atol=1e-14), "equal keys"
    # two tokens, scores ln 3 and 0: weights 3/4 and 1/4 (checks the scale and the sign).
    d2 = 4
    qv = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    scale = 0.5
    K2 = np.zeros((2, 1, d2), np.float32)
    K2[0, 0, 0] = np.float32(2 * math.log(3.0))          # scale * q.k0 = ln 3 (to float32)
    V2 = _f32(rng, 2, 1, d2)
    out = _single(oracle, qv, K2, V2, scale)
    s0 = scale * float(K2[0, 0, 0])
    w0 = math.exp(s0) / (math.exp(s0) + 1.0)
    assert abs(w0 - 0.75) < 1e-7
    want = w0 * V2[0, 0].astype(np.float64) + (1 - w0) * V2[1, 0].astype(np.float64)
    assert np.allclose(out[0], want, atol=1e-14), "3:1 split"
    # one dominant key: its value row, to float64 rounding.
    K3 = _f32(rng, 30, 1, d2) * np.float32(0.01)
    K3[13, 0, :] = np.float32(1000.0)
    V3 = _f32(rng, 30, 1, d2)
    q3 = np.ones((1, d2), np.float32)
    out = _single(oracle, q3, K3, V3, 1.0)
    assert np.allclose(out[0], V3[13, 0].astype(np.float64), atol=1e-12), "dominant key"
    # identical query heads in a group give identical outputs; other group differs.
    qi = np.repeat(_f32(rng, 1, d), 4, axis=0)
    K4, V4 = _f32(rng, 19, 2, d), _f32(rng, 19, 2, d)
    out = _single(oracle, qi, K4, V4, 0.35)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[2], out[3])
    assert not np.allclose(out[0], out[2])
    # L = 0 gives zeros (reading for an empty context).
    kc = np.full((4, 1, 2, BS, 4), np.nan, np.float32)
    vc = np.full((4, 1, 8, BS), np.nan, np.float32)
    out = oracle.decode(_f32(rng, 1, 2, 8), kc, vc, np.zeros((1, 1), np.int32),
                        np.zeros(1, np.int32), 0.3, BS, "f32")
    assert np.array_equal(out, np.zeros_like(out)), "L=0"


def pin_page_permutation(oracle):
    """Relabelling physical pages (and editing the table to match) changes nothing."""
    rng = np.random.default_rng(14)
    L, hq, hkv, d, nb = 75, 4, 2, 8, 10
    K, V, q = _f32(rng, L, hkv, d), _f32(rng, L, hkv, d), _f32(rng, 1, hq, d)
    table = [int(p) for p in rng.permutation(nb)[:5]]
    kc, vc = contiguous_to_paged(K, V, table, BS, nb, 4)
    base = oracle.decode(q, kc, vc, np.array([table], np.int32), np.array([L], np.int32),
                         0.3, BS, "f32")
    perm = rng.permutation(nb)                       # physical page p moves to perm[p]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    table2 = [int(perm[p]) for p in table]
    moved = oracle.decode(q, kc2, vc2, np.array([table2], np.int32), np.array([L], np.int32),
                          0.3, BS, "f32")
    assert np.array_equal(base, moved)
    # a bigger pool and NaN everywhere nobody reads change nothing either
    kc3 = np.full((nb + 7,) + kc.shape[1:], np.nan, np.float32)
    vc3 = np.full((nb + 7,) + vc.shape[1:], np.nan, np.float32)
    table3 = [p + 7 for p in table]
    pos = np.arange(L)
    for t in pos:
        p, o = table[t // BS], t % BS
        kc3[p + 7, :, :, o, :] = kc[p, :, :, o, :]
        vc3[p + 7, :, :, o] = vc[p, :, :, o]
    padded = np.array([table3 + [0, 1, 2]], np.int32)    # unused entries point at NaN pages
    far = oracle.decode(q, kc3, vc3, padded, np.array([L], np.int32), 0.3, BS, "f32")
    assert np.array_equal(base, far)


def pin_batch_rows(oracle):
    """Several sequences of different lengths in one pool and one call: row b
    is the brute force over sequence b's own contiguous tensor (so each row
    reads its own table row and length)."""
    rng = np.random.default_rng(15)
    lens, hq, hkv, d, bs, x = [23, 5, 40, 17], 4, 2, 8, 16, 4
    npg = [-(-L // bs) for L in lens]
    nb = sum(npg) + 1
    perm = [int(p) for p in rng.permutation(nb)]
    kc = np.full((nb, hkv, d // x, bs, x), np.nan, dtype=np.float32)
    vc = np.full((nb, hkv, d, bs), np.nan, dtype=np.float32)
    tables = np.full((len(lens), max(npg)), perm[-1], dtype=np.int32)
    seqs, at = [], 0
    for b, L in enumerate(lens):
        K, V = _f32(rng, L, hkv, d), _f32(rng, L, hkv, d)
        pages = perm[at:at + npg[b]]
        at += npg[b]
        tables[b, :npg[b]] = pages
        k1, v1 = contiguous_to_paged(K, V, pages, bs, nb, x)
        for p in pages:
            kc[p], vc[p] = k1[p], v1[p]
        seqs.append((K, V))
    q = _f32(rng, len(lens), hq, d)
    scale = float(np.float32(0.3))
    got = oracle.decode(q, kc, vc, tables, np.array(lens, np.int32), scale, bs, "f32")
    for b, (K, V) in enumerate(seqs):
        want = np.array(brute_attention(q[b].astype(np.float64).tolist(), K.astype(np.float64).tolist(),
                                        V.astype(np.float64).tolist(), scale, hq // hkv))
        assert np.allclose(got[b], want, rtol=0, atol=1e-12), b


ALL_PINS = [pin_brute_force, pin_library_sdpa, pin_closed_forms, pin_page_permutation, pin_batch_rows]
