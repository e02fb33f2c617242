"""Multi-query paged attention, plain definition in float64 (test
infrastructure only).

What is computed.  A step in which sequence ``b`` brings ``n_b`` new tokens
at once -- draft tokens to verify, or a chunk of a prompt -- whose K/V rows
are already written to the paged cache, so the sequence now holds
``L_b = context_lens[b]`` tokens, the new ones at positions
``L_b - n_b .. L_b - 1``.  The query of new token ``j`` attends over the
positions it may see, ``0 .. L_b - n_b + j``, through the block table,
exactly as a decode query does over its whole context.  The pages name this
case only as speculative decoding's kernels verifying parallel draft tokens
across paged memory [PagedAttention Internals, "The Mathematical Cause of
KV Cache Fragmentation", closing link]; the paging and the attention are
those of [PagedAttention Internals, "How PagedAttention Works" items 1-3].

Readings (listed in the design notes):
  * causal within the new tokens: token j sees the old context, the new
    tokens before it and itself, not the ones after it;
  * query rows are packed by sequence: rows ``query_start[b] ..
    query_start[b+1] - 1`` of ``q`` and of the output belong to sequence b,
    in position order; ``n_b <= L_b``;
  * everything else (GQA mapping, scale, layouts, storage dtypes) is that of
    ``oracle.decode``.
"""

import numpy as np

from .formats import to_f64
from .paged_attention import attend, gather_sequence, kv_head_of


def visible_positions(context_len: int, num_new: int, j: int) -> int:
    """Number of positions new token j of a sequence sees (its own included)."""
    return int(context_len) - int(num_new) + int(j) + 1


def decode_multi(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                 block_size: int, dtype: str, seqs=None) -> np.ndarray:
    """Reference output, float64 [num_tokens, heads, D] (rows of sequences not
    in ``seqs`` are left zero)."""
    T, hq, d = q.shape
    hkv = k_cache.shape[1]
    if hq % hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    scale = float(np.float32(scale))
    qs = [int(x) for x in query_start]
    B = len(qs) - 1
    seqs = range(B) if seqs is None else [int(s) for s in seqs]
    out = np.zeros((T, hq, d), dtype=np.float64)
    for b in seqs:
        n = qs[b + 1] - qs[b]
        L = int(context_lens[b])
        if n < 0 or n > L:
            raise ValueError(f"sequence {b}: {n} new tokens in a context of {L}")
        K, V = gather_sequence(k_cache, v_cache, block_tables[b], L, block_size, dtype)
        for j in range(n):
            row = qs[b] + j
            seen = visible_positions(L, n, j)
            qrow = to_f64(np.ascontiguousarray(q[row]), dtype)
            for h in range(hq):
                g = kv_head_of(h, group)
                out[row, h] = attend(qrow[h], K[:seen, g, :], V[:seen, g, :], scale)
    return out
