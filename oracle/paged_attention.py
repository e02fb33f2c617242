"""Paged decode attention, plain definition in float64 (test infrastructure only).

What is computed.  One decode step of one attention layer: sequence ``b`` has
``L = context_lens[b]`` tokens whose key and value vectors sit in fixed-size
pages of ``block_size`` tokens; its block table maps logical block ``i`` (the
tokens ``i*bs .. i*bs+bs-1``) to a physical page id, and token ``t`` lives in
page ``table[t // bs]`` at offset ``t % bs``.  [Glossary, "Technical
Architecture" and its page-table figure; Internals, "How PagedAttention
Works" items 1-2]  The kernel reads keys and values through that table and
runs scaled dot-product attention.  [Internals, "How PagedAttention Works"
item 3; Glossary, "On-the-Fly CUDA Block Fetching"]

Readings where the pages are silent (each listed in the design notes):
  * attention is softmax(scale * q . k_t) over all L cached tokens, then the
    weighted sum of v_t; no mask, bias or soft-cap; the newest token (already
    appended) attends to itself;
  * query head h uses kv head h // (num_heads / num_kv_heads);
  * L = 0 gives an all-zero output;
  * layouts: k_cache [blocks][kv_heads][head_dim/X][block_size][X] (X elements
    = 16 bytes), v_cache [blocks][kv_heads][head_dim][block_size],
    q [seqs][heads][head_dim];
  * ``scale`` is used as the exact float32 value given to the device.
Paging changes only where K/V are read from, never the result, so the value
computed here is the textbook attention of the gathered sequence.
"""

import numpy as np

from .formats import to_f64


def resolve_slot(table_row, pos: int, block_size: int):
    """Token position -> (physical page, offset inside the page)."""
    return int(table_row[pos // block_size]), pos % block_size


def gather_sequence(k_cache, v_cache, table_row, context_len: int, block_size: int,
                    dtype: str):
    """Read one sequence's keys and values through its block table.

    Returns float64 arrays K, V of shape [L, num_kv_heads, head_dim].
    Only the first ceil(L / block_size) table entries and the first L slots
    are touched.
    """
    L = int(context_len)
    nb, hkv, nchunk, bs, x = k_cache.shape
    if bs != block_size:
        raise ValueError("k_cache block axis does not match block_size")
    d = nchunk * x
    pos = np.arange(L)
    pages = np.asarray(table_row, dtype=np.int64)[pos // bs] if L else np.zeros(0, np.int64)
    offs = pos % bs
    k = k_cache[pages, :, :, offs, :]            # [L, hkv, D/X, X]
    v = v_cache[pages, :, :, offs]               # [L, hkv, D]
    K = to_f64(np.ascontiguousarray(k), dtype).reshape(L, hkv, d)
    V = to_f64(np.ascontiguousarray(v), dtype).reshape(L, hkv, d)
    return K, V


def kv_head_of(head: int, group: int) -> int:
    """Query head -> the kv head it reads (contiguous groups of ``group``)."""
    return head // group


def attend(qvec: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query vector (float64, exact inputs)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = float(scale) * (K @ qvec)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
           block_size: int, dtype: str, seqs=None) -> np.ndarray:
    """Reference output for the given sequences, float64 [len(seqs), heads, D].

    ``q``/caches are storage arrays: float32 for 'f32', uint16 patterns for
    'bf16'.  ``seqs`` selects a subset of sequences (default: all).
    """
    B, hq, d = q.shape
    hkv = k_cache.shape[1]
    if hq % hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    scale = float(np.float32(scale))
    seqs = range(B) if seqs is None else [int(s) for s in seqs]
    out = np.zeros((len(seqs), hq, d), dtype=np.float64)
    for i, b in enumerate(seqs):
        K, V = gather_sequence(k_cache, v_cache, block_tables[b], int(context_lens[b]),
                               block_size, dtype)
        qb = to_f64(np.ascontiguousarray(q[b]), dtype)
        for h in range(hq):
            g = kv_head_of(h, group)
            out[i, h] = attend(qb[h], K[:, g, :], V[:, g, :], scale)
    return out
