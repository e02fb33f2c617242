"""Host-side block manager used to build the block tables, slot mappings and
copy-on-write copy lists that the device kernels consume.

It is input plumbing, not part of the data-parallel path: it decides *where*
tokens live, the kernels then read and write those places.

Behaviour restated from the pages (own code, same observable behaviour):

* Pages of ``block_size`` tokens come from a pool of free physical page ids.
  A request for ``n`` tokens takes ceil(n / block_size) pages, taken from the
  front of the free list; too few free pages is an out-of-memory error.
  [What is PagedAttention? (esaholic glossary), "Step-by-Step Implementation
  Framework"; PagedAttention Internals (dailyaiworld), "Implementation: Custom
  Block Manager Simulation", block_manager.py allocate_sequence]
* Each page carries a reference count: 1 on allocation, raised when another
  sequence shares it, lowered on free; at zero the page goes to the back of
  the free list (so reuse is first-in first-out).
  [PagedAttention Internals, "Copy-on-Write and Prefix Sharing" and
  block_manager.py free_sequence; What is PagedAttention?, tradeoffs table,
  "Copy-on-Write Page Sharing" row]
* When a sequence grows by one token and that token opens a new block, one
  more page is taken from the pool, otherwise the token goes into the last
  page.  [PagedAttention Internals, "How PagedAttention Works" item 2 and
  block_manager.py append_token]
* Sequences forked from a parent share its pages (reference counts go up); a
  write into a shared page first moves the writer onto a fresh private copy.
  [What is PagedAttention?, "Copy-on-Write Memory Forking"; PagedAttention
  Internals, "Copy-on-Write and Prefix Sharing"]

Readings taken where the pages leave a step open:

* The listing's append trigger tests the token count modulo the block size
  against 1; we read the count as the sequence length *after* the new token,
  so a page is taken exactly when the new token's position is a multiple of
  the block size.
* A physical slot is ``page * block_size + offset``.
* Copy-on-write copies only while the page is still shared (reference count
  above one); the last holder of a formerly shared page writes in place.
"""

from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Tuple


class OutOfPages(MemoryError):
    """The free pool cannot satisfy an allocation."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("num_blocks must be >= 0 and block_size > 0")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.free: deque = deque(order)
        self.ref = [0] * num_blocks
        self.tables: Dict[object, List[int]] = {}
        self.lengths: Dict[object, int] = {}
        # (src, dst) page copies requested by copy-on-write, in issue order.
        self.pending_copies: List[Tuple[int, int]] = []

    # -- pool -------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def _take(self) -> int:
        if not self.free:
            raise OutOfPages("no free physical pages left")
        page = self.free.popleft()
        self.ref[page] = 1
        return page

    def _release(self, page: int) -> None:
        self.ref[page] -= 1
        if self.ref[page] < 0:
            raise RuntimeError(f"page {page} released more often than taken")
        if self.ref[page] == 0:
            self.free.append(page)

    # -- sequences --------------------------------------------------------
    def blocks_for(self, num_tokens: int) -> int:
        return -(-int(num_tokens) // self.block_size)

    def allocate(self, seq, num_tokens: int) -> List[int]:
        """Give ``seq`` room for ``num_tokens`` tokens (all pages up front)."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq!r} already exists")
        if num_tokens < 0:
            raise ValueError("num_tokens must be >= 0")
        need = self.blocks_for(num_tokens)
        if need > len(self.free):
            raise OutOfPages(f"need {need} pages, {len(self.free)} free")
        pages = [self._take() for _ in range(need)]
        self.tables[seq] = pages
        self.lengths[seq] = int(num_tokens)
        return list(pages)

    def slot(self, seq, pos: int) -> int:
        """Physical slot of token ``pos`` of ``seq``."""
        if not 0 <= pos < self.lengths[seq]:
            raise IndexError(f"position {pos} outside sequence of length {self.lengths[seq]}")
        page = self.tables[seq][pos // self.block_size]
        return page * self.block_size + pos % self.block_size

    def append_token(self, seq) -> int:
        """Grow ``seq`` by one token and return the slot the token goes to.

        Takes a new page when the token opens a block; moves the sequence onto
        a private copy of its last page first when that page is shared.
        """
        table = self.tables[seq]
        pos = self.lengths[seq]
        if pos % self.block_size == 0:
            table.append(self._take())
        else:
            last = table[-1]
            if self.ref[last] > 1:
                fresh = self._take()
                self.pending_copies.append((last, fresh))
                self._release(last)
                table[-1] = fresh
        self.lengths[seq] = pos + 1
        return table[-1] * self.block_size + pos % self.block_size

    def fork(self, parent, child) -> None:
        """``child`` starts as ``parent``: same pages, shared by reference."""
        if child in self.tables:
            raise KeyError(f"sequence {child!r} already exists")
        pages = list(self.tables[parent])
        for p in pages:
            self.ref[p] += 1
        self.tables[child] = pages
        self.lengths[child] = self.lengths[parent]

    def free_sequence(self, seq) -> None:
        """Drop ``seq``; pages nobody else holds go back to the free list."""
        pages = self.tables.pop(seq, None)
        if pages is None:
            return
        del self.lengths[seq]
        for p in pages:
            self._release(p)

    def take_copies(self) -> List[Tuple[int, int]]:
        out, self.pending_copies = self.pending_copies, []
        return out
