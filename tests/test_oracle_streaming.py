"""The chunked online softmax and the partition/merge algebra agree with the
plain definition in float64 (pins the split path's algebra, CPU only)."""

import numpy as np
import pytest

import oracle
from oracle.paged_attention import attend


def _case(seed, L, hq, hkv, d, spread=1.0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L, hkv, d)) * spread
    V = rng.standard_normal((L, hkv, d))
    q = rng.standard_normal((hq, d))
    return q, K, V


def _plain(q, K, V, scale, group):
    return np.stack([attend(q[h], K[:, h // group], V[:, h // group], scale) for h in range(q.shape[0])])


@pytest.mark.parametrize("L,chunk", [(1, 32), (31, 32), (32, 32), (33, 32), (517, 32), (1000, 16), (2049, 64)])
def test_online_equals_plain(L, chunk):
    q, K, V = _case(L, L, 8, 2, 16, spread=3.0)
    got = oracle.online_decode_sequence(q, K, V, 0.2, 4, chunk)
    assert np.allclose(got, _plain(q, K, V, 0.2, 4), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,part", [(1, 512), (511, 512), (512, 512), (513, 512), (5000, 512), (32768, 512), (3000, 256)])
def test_split_merge_equals_plain(L, part):
    q, K, V = _case(L + 1, L, 4, 1, 8, spread=2.0)
    got = oracle.split_decode_sequence(q, K, V, 0.3, 4, part, 32)
    assert np.allclose(got, _plain(q, K, V, 0.3, 4), rtol=0, atol=1e-12)


def test_split_with_wildly_different_partition_maxima():
    """Partitions whose maxima differ by ~700 (e^-700 ~ 1e-304) still merge."""
    q, K, V = _case(9, 1024, 1, 1, 4)
    K[:512] *= 0.0
    K[700] = q[0] * 200.0     # one partition holds a score ~ 700 above the rest
    got = oracle.split_decode_sequence(q, K, V, 1.0, 1, 512, 32)
    assert np.allclose(got, _plain(q, K, V, 1.0, 1), rtol=0, atol=1e-12)
    assert np.allclose(got[0], V[700, 0], atol=1e-12)


def test_empty_context_gives_zeros():
    q, K, V = _case(3, 0, 2, 1, 4)
    assert not oracle.split_decode_sequence(q, K, V, 1.0, 2, 512, 32).any()
    assert not oracle.online_decode_sequence(q, K, V, 1.0, 2, 32).any()


def _shared_prefix_cuts(S, P, L):
    """Segments of the shared-prefix path: the prefix [0, S) in partitions of
    P (the last one cut at S), then the rest [S, L) on the partition grid."""
    cuts = list(range(0, S, P)) + [S]
    cuts += [c for c in range(P * (S // P + 1), L, P)] + [L]
    return sorted(set(cuts))


@pytest.mark.parametrize("L,S,P", [(1000, 640, 256), (1000, 768, 256), (10512, 9984, 2048), (100, 96, 64),
                                   (100, 16, 64), (200, 192, 32), (50, 0, 32), (64, 64, 32), (65, 48, 32)])
def test_segments_cut_at_a_shared_prefix_equal_plain(L, S, P):
    q, K, V = _case(L + S, L, 8, 2, 16, spread=2.0)
    cuts = _shared_prefix_cuts(S, P, L)
    assert cuts[0] == 0 and cuts[-1] == L and all(b >= a for a, b in zip(cuts, cuts[1:]))
    if 0 < S < L:
        assert S in cuts
    got = oracle.segmented_decode_sequence(q, K, V, 0.25, 4, cuts, 32)
    assert np.allclose(got, _plain(q, K, V, 0.25, 4), rtol=0, atol=1e-12)


def test_segments_with_an_empty_one_and_uneven_cuts():
    q, K, V = _case(3, 300, 4, 1, 8, spread=3.0)
    for cuts in ([0, 0, 300], [0, 7, 7, 150, 299, 300], [0, 1, 2, 3, 300], [0, 300, 300]):
        got = oracle.segmented_decode_sequence(q, K, V, 0.3, 4, cuts, 32)
        assert np.allclose(got, _plain(q, K, V, 0.3, 4), rtol=0, atol=1e-12), cuts


def test_overlapping_segments_are_caught():
    """The mistake a per-sequence launch that ignored the shared length would
    make -- reading the partly shared partition from its start, so positions
    kP .. S - 1 count twice -- gives a different result."""
    L, S, P = 1000, 640, 256
    q, K, V = _case(5, L, 8, 2, 16, spread=2.0)
    good = oracle.segmented_decode_sequence(q, K, V, 0.25, 4, _shared_prefix_cuts(S, P, L), 32)
    # prefix segments [0,256) [256,512) [512,640) plus the rest read from 512 again
    hq, d = q.shape
    bad = np.zeros((hq, d))
    for h in range(hq):
        g = h // 4
        segs = [(0, 256), (256, 512), (512, 640), (512, 768), (768, 1000)]
        parts = [oracle.streaming._online(q[h], K[a:b, g], V[a:b, g], 0.25, 32) for a, b in segs]
        M = max(p[0] for p in parts)
        w = [np.exp(p[0] - M) for p in parts]
        bad[h] = sum(wi * p[2] for wi, p in zip(w, parts)) / sum(wi * p[1] for wi, p in zip(w, parts))
    assert np.abs(bad - _plain(q, K, V, 0.25, 4)).max() > 1e-3
    assert np.allclose(good, _plain(q, K, V, 0.25, 4), rtol=0, atol=1e-12)
