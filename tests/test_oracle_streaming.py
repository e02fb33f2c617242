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
