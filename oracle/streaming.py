"""Streaming forms of the same attention, in float64 (test infrastructure only).

A decode kernel cannot hold all L scores at once; it walks the context in
chunks, keeping per query head a running maximum ``m``, a running sum ``l``
of exp(score - m) and an accumulator ``acc`` of exp(score - m)-weighted value
rows, rescaling both by exp(m_old - m_new) whenever the maximum grows.  Long
contexts are further cut into partitions processed independently; partition
``p`` leaves (m_p, l_p, acc_p) and a second pass merges them with
M = max_p m_p, out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p.

Both are exact rearrangements of softmax(s) V (the common factor e^-M
cancels), so in float64 they must agree with the plain definition to
rounding.  This module writes the algebra out step by step so the tests can
check it against the plain definition; the device kernels are written
separately and only their outputs are compared.
"""

import numpy as np


def _online(qvec, K, V, scale, chunk):
    m, l = -np.inf, 0.0
    acc = np.zeros(V.shape[1], dtype=np.float64)
    for start in range(0, K.shape[0], chunk):
        s = scale * (K[start:start + chunk] @ qvec)
        m_new = max(m, float(s.max()))
        alpha = np.exp(m - m_new)            # 0 on the first chunk (m = -inf)
        p = np.exp(s - m_new)
        l = l * alpha + float(p.sum())
        acc = acc * alpha + p @ V[start:start + chunk]
        m = m_new
    return m, l, acc


def online_decode_sequence(qb, K, V, scale: float, group: int, chunk: int):
    """Chunked online-softmax attention for every head of one sequence."""
    hq, d = qb.shape
    out = np.zeros((hq, d), dtype=np.float64)
    if K.shape[0] == 0:
        return out
    for h in range(hq):
        g = h // group
        m, l, acc = _online(qb[h], K[:, g, :], V[:, g, :], scale, chunk)
        out[h] = acc / l
    return out


def split_decode_sequence(qb, K, V, scale: float, group: int, partition: int, chunk: int):
    """Partitioned attention plus the merge pass, for one sequence."""
    hq, d = qb.shape
    out = np.zeros((hq, d), dtype=np.float64)
    L = K.shape[0]
    if L == 0:
        return out
    for h in range(hq):
        g = h // group
        parts = [_online(qb[h], K[s:s + partition, g, :], V[s:s + partition, g, :], scale, chunk)
                 for s in range(0, L, partition)]
        M = max(p[0] for p in parts)
        w = [np.exp(p[0] - M) for p in parts]
        num = sum(wi * p[2] for wi, p in zip(w, parts))
        den = sum(wi * p[1] for wi, p in zip(w, parts))
        out[h] = num / den
    return out


def segmented_decode_sequence(qb, K, V, scale: float, group: int, cuts, chunk: int):
    """Attention over consecutive segments [cuts[i], cuts[i + 1]) of one
    sequence's context, each reduced to (m, l, acc) on its own and merged as
    the partitions are.  The cuts need not be equally spaced: a prefix shared
    by several sequences can end inside a partition, and the partition is
    then read as two segments.  An empty segment leaves m = -inf, l = 0 and
    weighs nothing in the merge."""
    hq, d = qb.shape
    out = np.zeros((hq, d), dtype=np.float64)
    if K.shape[0] == 0:
        return out
    cuts = list(cuts)
    for h in range(hq):
        g = h // group
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if b > a:
                parts.append(_online(qb[h], K[a:b, g, :], V[a:b, g, :], scale, chunk))
            else:
                parts.append((-np.inf, 0.0, np.zeros(d, dtype=np.float64)))
        M = max(p[0] for p in parts)
        w = [np.exp(p[0] - M) if p[0] > -np.inf else 0.0 for p in parts]
        num = sum(wi * p[2] for wi, p in zip(w, parts))
        den = sum(wi * p[1] for wi, p in zip(w, parts))
        out[h] = num / den
    return out
