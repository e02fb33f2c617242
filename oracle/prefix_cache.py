"""Page reuse by prompt content (prefix caching) -- TEST INFRASTRUCTURE ONLY.

A plain model of a page pool whose prompts share their leading full pages
with earlier prompts of the same content [Paged Attention (AI terminology),
"Key Points" (sharing row) and "Common Usage Examples" (prefix caching);
PagedAttention Internals, "Copy-on-Write and Prefix Sharing" and
"Architectural Recommendations" item 2].  The pages say only that requests
with the same prefix point at the same physical pages and that the pages'
reference counts rise; the readings taken here:

* a full page is identified by the entire token prefix that ends with it
  (its K/V depends on every earlier token) -- no hashing: every distinct
  prefix gets its own integer id, interned from the pair (id of the prefix
  one page shorter, this page's tokens), so by induction two ids are equal
  exactly when the whole prefixes are; a partly filled page is never shared
  this way;
* a prompt shares the longest leading run of pages whose prefixes are
  registered, and registers each fresh full page under its prefix,
  replacing an older page registered under the same prefix;
* a registered page stays registered after its last holder frees it and
  goes back to the free list, and is dropped from the registry when the
  free list hands it out again; a hit on such a free page takes it back off
  the free list.

The rest (FIFO free list, reference counts, fork, copy-on-write on append,
free) is the pool the kernels' inputs come from, restated here so this file
stands alone.  Slow on purpose: lists, tuples and dicts.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class OutOfPages(MemoryError):
    pass


class PrefixCachingPool:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self.block_size = int(block_size)
        self.free: List[int] = list(range(num_blocks)) if free_order is None else [int(p) for p in free_order]
        self.ref = [0] * int(num_blocks)
        self.pages: Dict[int, List[int]] = {}
        self.length: Dict[int, int] = {}
        self.page_of: Dict[int, int] = {}      # prefix id -> page
        self.prefix_of: Dict[int, int] = {}    # page -> prefix id
        self.ids: Dict[Tuple[int, Tuple[int, ...]], int] = {}   # (shorter prefix id, page) -> id
        self.copies: List[Tuple[int, int]] = []

    # -- pool ------------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfPages
        page = self.free.pop(0)
        if page in self.prefix_of:                      # handed out again: evicted
            del self.page_of[self.prefix_of.pop(page)]
        self.ref[page] = 1
        return page

    def _release(self, page: int) -> None:
        self.ref[page] -= 1
        if self.ref[page] == 0:
            self.free.append(page)

    def prefix_ids(self, toks: Tuple[int, ...]) -> List[int]:
        """Id of toks[:(k + 1) * block_size] for every full page k (0 is the
        empty prefix)."""
        bs, out, prev = self.block_size, [], 0
        for k in range(len(toks) // bs):
            prev = self.ids.setdefault((prev, toks[k * bs:(k + 1) * bs]), len(self.ids) + 1)
            out.append(prev)
        return out

    def _register(self, page: int, prefix: int) -> None:
        old = self.page_of.get(prefix)
        if old is not None:
            del self.prefix_of[old]
        self.page_of[prefix] = page
        self.prefix_of[page] = prefix

    # -- sequences -------------------------------------------------------
    def allocate_prompt(self, seq: int, tokens: Sequence[int]) -> Tuple[List[int], int]:
        """Pages for a prompt and the number of leading tokens already cached."""
        if seq in self.pages:
            raise ValueError("sequence exists")
        toks = tuple(int(t) for t in tokens)
        bs = self.block_size
        full = len(toks) // bs
        total = -(-len(toks) // bs)
        keys = self.prefix_ids(toks)
        hits = []
        for k in range(full):
            page = self.page_of.get(keys[k])
            if page is None:
                break
            hits.append(page)
        taken_back = [p for p in hits if self.ref[p] == 0]
        if len(taken_back) + total - len(hits) > len(self.free):
            raise OutOfPages
        for p in taken_back:
            self.free.remove(p)
        pages = []
        for p in hits:
            self.ref[p] += 1
            pages.append(p)
        for k in range(len(hits), total):
            p = self._take()
            pages.append(p)
            if k < full:
                self._register(p, keys[k])
        self.pages[seq] = pages
        self.length[seq] = len(toks)
        return list(pages), len(hits) * bs

    def allocate(self, seq: int, num_tokens: int) -> List[int]:
        """A sequence whose pages are not registered (no token ids)."""
        if seq in self.pages:
            raise ValueError("sequence exists")
        need = -(-int(num_tokens) // self.block_size)
        if need > len(self.free):
            raise OutOfPages
        self.pages[seq] = [self._take() for _ in range(need)]
        self.length[seq] = int(num_tokens)
        return list(self.pages[seq])

    def fork(self, parent: int, child: int) -> None:
        if child in self.pages:
            raise ValueError("sequence exists")
        self.pages[child] = list(self.pages[parent])
        self.length[child] = self.length[parent]
        for p in self.pages[child]:
            self.ref[p] += 1

    def append_token(self, seq: int) -> int:
        """One more token: a fresh page when it opens a block, a private copy
        first when the last page is shared.  Returns the token's slot."""
        bs = self.block_size
        pages, pos = self.pages[seq], self.length[seq]
        if pos % bs == 0:
            pages.append(self._take())
        elif self.ref[pages[-1]] > 1:
            fresh = self._take()
            self.copies.append((pages[-1], fresh))
            self._release(pages[-1])
            pages[-1] = fresh
        self.length[seq] = pos + 1
        return pages[-1] * bs + pos % bs

    def free_sequence(self, seq: int) -> None:
        for p in self.pages.pop(seq, []):
            self._release(p)
        self.length.pop(seq, None)

    def cached_pages(self) -> List[int]:
        return sorted(self.prefix_of)
