"""The multi-query oracle (oracle/multi_query.py) pinned to things other than
itself, on the CPU:

* library     -- torch's scaled_dot_product_attention in float64: with
                 is_causal when the new tokens are the whole context (its own
                 causal convention), with an explicit boolean mask otherwise;
* brute force -- the pure-Python attention loop of the decode pins, run on
                 each query's visible prefix of a contiguous tensor;
* special case -- one new token per sequence is the (separately pinned)
                 decode oracle;
* invariants  -- a query's output ignores every later position, even NaN.

Each planted mistake (no causal mask, the mask aligned to the start instead
of the end, a strict mask that hides the token from itself, rows in the
wrong order) must fail one of these pins."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.multi_query as mq
from oracle_pins import brute_attention, contiguous_to_paged


def _case(rng, lens, news, hq, hkv, d, bs, x=4, extra_pages=3):
    """Contiguous K/V per sequence, scattered into one paged pool; q rows for
    the new tokens packed by sequence."""
    need = sum(-(-L // bs) for L in lens) + extra_pages
    perm = [int(p) for p in rng.permutation(need)]
    width = max(-(-L // bs) for L in lens) + 1
    tables = np.full((len(lens), width), perm[-1], dtype=np.int32)
    kc = np.full((need, hkv, d // x, bs, x), np.nan, dtype=np.float32)
    vc = np.full((need, hkv, d, bs), np.nan, dtype=np.float32)
    Ks, Vs, at = [], [], 0
    for b, L in enumerate(lens):
        K = rng.standard_normal((L, hkv, d)).astype(np.float32)
        V = rng.standard_normal((L, hkv, d)).astype(np.float32)
        pages = perm[at:at + -(-L // bs)]
        at += len(pages)
        tables[b, :len(pages)] = pages
        k1, v1 = contiguous_to_paged(K, V, pages or [0], bs, need, x)
        for p in pages:
            kc[p], vc[p] = k1[p], v1[p]
        Ks.append(K)
        Vs.append(V)
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), hq, d)).astype(np.float32)
    return q, Ks, Vs, kc, vc, tables, np.array(lens, np.int32), qs


def _sdpa(qrows, K, V, scale, mask=None, causal=False):
    """torch SDPA, float64, GQA by enable_gqa; qrows [n, hq, d], K/V [L, hkv, d]."""
    n, hq, d = qrows.shape
    tq = torch.from_numpy(qrows.astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
    tk = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
    tv = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).unsqueeze(0).contiguous()
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal,
                                                         scale=scale, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def pin_square_is_library_causal(orc):
    """All of a sequence's tokens are new (a prompt processed at once): torch's
    own causal attention."""
    rng = np.random.default_rng(21)
    bs = 16
    for L, hq, hkv, d in [(1, 2, 1, 8), (17, 4, 2, 8), (33, 8, 2, 16), (48, 6, 3, 8)]:
        q, Ks, Vs, kc, vc, tab, lens, qs = _case(rng, [L], [L], hq, hkv, d, bs)
        scale = float(np.float32(1 / math.sqrt(d)))
        got = orc.decode_multi(q, kc, vc, tab, lens, qs, scale, bs, "f32")
        want = _sdpa(q, Ks[0], Vs[0], scale, causal=True)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (L, np.abs(got - want).max())


def pin_library_end_aligned_mask(orc):
    """n < L new tokens: torch SDPA with the mask 'position t visible to new
    token j iff t <= L - n + j' (the causal band ends at the diagonal of the
    last query and the last key)."""
    rng = np.random.default_rng(22)
    lens, news = [40, 5, 77, 16, 33], [3, 5, 8, 1, 0]
    hq, hkv, d, bs = 8, 2, 16, 16
    q, Ks, Vs, kc, vc, tab, lens_a, qs = _case(rng, lens, news, hq, hkv, d, bs)
    scale = 0.3
    got = orc.decode_multi(q, kc, vc, tab, lens_a, qs, scale, bs, "f32")
    for b, (L, n) in enumerate(zip(lens, news)):
        if n == 0:
            continue
        mask = np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None]
        want = _sdpa(q[qs[b]:qs[b + 1]], Ks[b], Vs[b], float(np.float32(scale)), mask=mask)
        assert np.allclose(got[qs[b]:qs[b + 1]], want, rtol=0, atol=1e-12), b


def pin_brute_force(orc):
    rng = np.random.default_rng(23)
    lens, news = [9, 20, 3], [2, 4, 3]
    hq, hkv, d, bs = 4, 2, 4, 16
    q, Ks, Vs, kc, vc, tab, lens_a, qs = _case(rng, lens, news, hq, hkv, d, bs)
    scale = float(np.float32(0.41))
    got = orc.decode_multi(q, kc, vc, tab, lens_a, qs, scale, bs, "f32")
    for b, (L, n) in enumerate(zip(lens, news)):
        for j in range(n):
            seen = L - n + j + 1
            want = brute_attention(q[qs[b] + j].astype(np.float64).tolist(),
                                   Ks[b][:seen].astype(np.float64).tolist(),
                                   Vs[b][:seen].astype(np.float64).tolist(), scale, hq // hkv)
            assert np.allclose(got[qs[b] + j], np.array(want), rtol=0, atol=1e-12), (b, j)


def pin_one_new_token_is_decode(orc):
    rng = np.random.default_rng(24)
    lens = [36, 42, 1, 100]
    hq, hkv, d, bs = 8, 4, 8, 32
    q, Ks, Vs, kc, vc, tab, lens_a, qs = _case(rng, lens, [1] * 4, hq, hkv, d, bs)
    got = orc.decode_multi(q, kc, vc, tab, lens_a, qs, 0.25, bs, "f32")
    want = oracle.decode(q, kc, vc, tab, lens_a, 0.25, bs, "f32")
    assert np.array_equal(got, want)


def pin_later_positions_are_ignored(orc):
    """Poison K/V of the last new token with NaN: every earlier query of that
    sequence is unchanged (and finite)."""
    rng = np.random.default_rng(25)
    lens, news = [30, 50], [6, 4]
    hq, hkv, d, bs = 4, 4, 8, 16
    q, Ks, Vs, kc, vc, tab, lens_a, qs = _case(rng, lens, news, hq, hkv, d, bs)
    base = orc.decode_multi(q, kc, vc, tab, lens_a, qs, 0.3, bs, "f32")
    for b, L in enumerate(lens):
        kc2, vc2 = kc.copy(), vc.copy()
        page, off = tab[b][(L - 1) // bs], (L - 1) % bs
        kc2[page, :, :, off, :] = np.nan
        vc2[page, :, :, off] = np.nan
        got = orc.decode_multi(q, kc2, vc2, tab, lens_a, qs, 0.3, bs, "f32")
        rows = slice(qs[b], qs[b + 1] - 1)
        assert np.isfinite(got[rows]).all() and np.array_equal(got[rows], base[rows]), b


ALL = [pin_square_is_library_causal, pin_library_end_aligned_mask, pin_brute_force,
       pin_one_new_token_is_decode, pin_later_positions_are_ignored]


@pytest.mark.parametrize("pin", ALL, ids=lambda f: f.__name__)
def test_oracle_multi_query_pin(pin):
    pin(mq)


def test_rejects_more_new_tokens_than_context():
    rng = np.random.default_rng(26)
    q, Ks, Vs, kc, vc, tab, lens, qs = _case(rng, [4], [4], 2, 1, 4, 16)
    with pytest.raises(ValueError):
        mq.decode_multi(q, kc, vc, tab, np.array([3], np.int32), qs, 0.5, 16, "f32")


# -- planted mistakes -------------------------------------------------------------

class _Mutant:
    """The oracle module with one function swapped."""

    def __init__(self, **over):
        self.over = over

    def decode_multi(self, *args, **kw):
        saved = {k: getattr(mq, k) for k in self.over}
        try:
            for k, v in self.over.items():
                setattr(mq, k, v)
            return mq.decode_multi(*args, **kw)
        finally:
            for k, v in saved.items():
                setattr(mq, k, v)


def _reversed_rows(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, bs, dtype):
    out = mq.decode_multi(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, bs, dtype)
    fixed = out.copy()
    for b in range(len(query_start) - 1):
        a, e = int(query_start[b]), int(query_start[b + 1])
        fixed[a:e] = out[a:e][::-1]
    return fixed


class _RowOrder:
    decode_multi = staticmethod(_reversed_rows)


MUTANTS = {
    "no_causal_mask": _Mutant(visible_positions=lambda L, n, j: int(L)),
    "start_aligned": _Mutant(visible_positions=lambda L, n, j: int(j) + 1),
    "strict_mask": _Mutant(visible_positions=lambda L, n, j: int(L) - int(n) + int(j)),
    "rows_reversed": _RowOrder(),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    m = MUTANTS[name]
    caught = []
    for pin in ALL:
        try:
            pin(m)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, name
