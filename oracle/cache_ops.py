"""KV-append scatter and page copy, bit-exact definitions (test infrastructure only).

Both operate on storage arrays and move bits only (no arithmetic on values):
float32 arrays are handled through a uint32 view, bf16 data is uint16
patterns, so NaN payloads survive unchanged.

* Append: new token ``i`` goes to slot ``s = slot_mapping[i]``, i.e. page
  ``s // bs`` offset ``s % bs``; a negative slot means "no write".  Its key row
  fills k_cache[page, :, :, off, :] (head_dim split in 16-byte chunks) and its
  value row v_cache[page, :, :, off].  [Internals, "How PagedAttention Works"
  item 2 (pages taken on demand as tokens are generated); Glossary, page-table
  figure for the slot arithmetic]
* Page copy (copy-on-write fork): every (src, dst) pair makes page ``dst`` an
  exact copy of page ``src`` (all kv heads, K and V).  Pairs act as if applied
  at once, from the pages' contents before the call.  [Glossary,
  "Copy-on-Write Memory Forking"; Internals, "Copy-on-Write and Prefix
  Sharing"]
"""

import numpy as np


def _bits(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype in (np.uint16, np.uint32):
        return a
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, block_size: int):
    """Return copies of (k_cache, v_cache) with the new rows scattered in."""
    kc = _bits(k_cache).copy()
    vc = _bits(v_cache).copy()
    kn = _bits(k_new)
    vn = _bits(v_new)
    nb, hkv, nchunk, bs, x = kc.shape
    if bs != block_size:
        raise ValueError("k_cache block axis does not match block_size")
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        page, off = divmod(int(slot), bs)
        kc[page, :, :, off, :] = kn[i].reshape(hkv, nchunk, x)
        vc[page, :, :, off] = vn[i]
    if np.asarray(k_cache).dtype == np.float32:
        return kc.view(np.float32), vc.view(np.float32)
    return kc, vc


def copy_blocks(k_cache, v_cache, pairs):
    """Return copies of (k_cache, v_cache) after the page copies."""
    kb, vb = _bits(k_cache), _bits(v_cache)
    kc, vc = kb.copy(), vb.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        kc[dst] = kb[src]
        vc[dst] = vb[src]
    if np.asarray(k_cache).dtype == np.float32:
        return kc.view(np.float32), vc.view(np.float32)
    return kc, vc
