"""Thin binding over the native page allocator in libpa.so (include/pa_blockmgr.h).

Argument marshalling only: every decision -- which page a token gets, when a
block opens, when copy-on-write copies -- is made by the C++ code.  Method
names follow the host block manager the workloads use, so either can drive
the same code.  Sequence ids are Python ints (int64).
"""

from __future__ import annotations

import ctypes
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from . import _binding as B

_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p

_SIGNATURES = {
    "pa_bm_create": ([_i64, _i32, _vp, ctypes.POINTER(_vp)], _i32),
    "pa_bm_destroy": ([_vp], None),
    "pa_bm_num_free": ([_vp], _i64),
    "pa_bm_num_seqs": ([_vp], _i64),
    "pa_bm_seq_len": ([_vp, _i64], _i64),
    "pa_bm_seq_pages": ([_vp, _i64, _i64, _vp], _i64),
    "pa_bm_ref_count": ([_vp, _i64], _i32),
    "pa_bm_free_list": ([_vp, _i64, _vp], _i64),
    "pa_bm_allocate": ([_vp, _i64, _i64], _i32),
    "pa_bm_allocate_prompt": ([_vp, _i64, _vp, _i64, ctypes.POINTER(_i64)], _i32),
    "pa_bm_num_cached": ([_vp], _i64),
    "pa_bm_page_cached": ([_vp, _i64], _i32),
    "pa_bm_fork": ([_vp, _i64, _i64], _i32),
    "pa_bm_free": ([_vp, _i64], _i32),
    "pa_bm_append": ([_vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp], _i32),
    "pa_bm_block_tables": ([_vp, _vp, _i32, _i32, _i32, _vp, _vp], _i32),
    "pa_bm_shared_prefix": ([_vp, _vp, _i32], _i64),
    "pa_bm_prefix_groups": ([_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp], _i32),
}

PA_ERR_OUT_OF_PAGES, PA_ERR_NOT_FOUND, PA_ERR_HOST_MEMORY = -6, -7, -8

_configured = False


def _lib():
    global _configured
    lib = B.lib()
    if not _configured:
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _configured = True
    return lib


class OutOfPages(MemoryError):
    """The page pool cannot satisfy the request (nothing was taken)."""


def _check(fn: str, status: int) -> None:
    if status == 0:
        return
    msg = B.status_string(status)
    if status == PA_ERR_OUT_OF_PAGES:
        raise OutOfPages(f"{fn}: {msg}")
    if status == PA_ERR_NOT_FOUND:
        raise KeyError(f"{fn}: {msg}")
    raise B.PaError(fn, status, msg)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class NativeBlockManager:
    """Page pool of ``num_blocks`` pages of ``block_size`` tokens."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Iterable[int]] = None):
        lib = _lib()
        handle = _vp()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(list(free_order), dtype=np.int64))
            if order.shape != (num_blocks,):
                raise ValueError("free_order must list every page once")
        st = lib.pa_bm_create(int(num_blocks), int(block_size),
                              _ptr(order) if order is not None else None, ctypes.byref(handle))
        if st != 0:
            if st == -2:
                raise ValueError("invalid pool (sizes, or free_order is not a permutation)")
            _check("pa_bm_create", st)
        self._h = handle
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.pending_copies: List[Tuple[int, int]] = []

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- views matching the host block manager the workloads use ----------
    class _Tables:
        def __init__(self, mgr):
            self._m = mgr

        def __getitem__(self, seq):
            return self._m.pages(seq)

        def __contains__(self, seq):
            return int(_lib().pa_bm_seq_len(self._m._h, int(seq))) >= 0

    @property
    def tables(self):
        """Read-only mapping seq -> page list."""
        return NativeBlockManager._Tables(self)

    @property
    def free(self) -> List[int]:
        """The free list, front first."""
        return self.free_list()

    # -- queries ---------------------------------------------------------
    def num_free(self) -> int:
        return int(_lib().pa_bm_num_free(self._h))

    def num_seqs(self) -> int:
        return int(_lib().pa_bm_num_seqs(self._h))

    def length(self, seq: int) -> int:
        n = int(_lib().pa_bm_seq_len(self._h, int(seq)))
        if n < 0:
            raise KeyError(seq)
        return n

    def pages(self, seq: int) -> List[int]:
        lib = _lib()
        n = int(lib.pa_bm_seq_pages(self._h, int(seq), 0, None))
        if n < 0:
            raise KeyError(seq)
        out = np.zeros(max(n, 1), dtype=np.int32)
        lib.pa_bm_seq_pages(self._h, int(seq), n, _ptr(out))
        return out[:n].tolist()

    def ref_count(self, page: int) -> int:
        return int(_lib().pa_bm_ref_count(self._h, int(page)))

    def free_list(self) -> List[int]:
        lib = _lib()
        n = int(lib.pa_bm_free_list(self._h, 0, None))
        out = np.zeros(max(n, 1), dtype=np.int32)
        lib.pa_bm_free_list(self._h, n, _ptr(out))
        return out[:n].tolist()

    # -- updates ---------------------------------------------------------
    def allocate(self, seq: int, num_tokens: int, return_pages: bool = True) -> Optional[List[int]]:
        st = _lib().pa_bm_allocate(self._h, int(seq), int(num_tokens))
        if st == -2:
            raise ValueError(f"sequence {seq} exists or num_tokens < 0")
        _check("pa_bm_allocate", st)
        return self.pages(seq) if return_pages else None

    def allocate_prompt(self, seq: int, tokens: Sequence[int], return_pages: bool = True):
        """New sequence for a prompt of token ids, sharing every leading full
        page an earlier prompt with the same prefix stored.  Returns (pages,
        number of leading tokens whose K/V is already cached); with
        return_pages=False only the count (the pages stay readable through
        pages() and block_tables())."""
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        cached = _i64(0)
        st = _lib().pa_bm_allocate_prompt(self._h, int(seq), _ptr(toks) if toks.size else None,
                                          int(toks.size), ctypes.byref(cached))
        if st == -2:
            raise ValueError(f"sequence {seq} exists")
        _check("pa_bm_allocate_prompt", st)
        if not return_pages:
            return int(cached.value)
        return self.pages(seq), int(cached.value)

    def num_cached(self) -> int:
        """Pages registered in the prefix cache (held or free)."""
        return int(_lib().pa_bm_num_cached(self._h))

    def is_cached(self, page: int) -> bool:
        return int(_lib().pa_bm_page_cached(self._h, int(page))) == 1

    def fork(self, parent: int, child: int) -> None:
        st = _lib().pa_bm_fork(self._h, int(parent), int(child))
        if st == -2:
            raise ValueError(f"sequence {child} exists")
        _check("pa_bm_fork", st)

    def free_sequence(self, seq: int) -> None:
        _check("pa_bm_free", _lib().pa_bm_free(self._h, int(seq)))

    def append(self, seqs: Sequence[int], tables: Optional[np.ndarray] = None,
               context_lens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        """One token for each of ``seqs`` (in order): returns (slots [n] int64,
        copy-on-write pairs [k, 2] int64).  ``tables`` / ``context_lens``
        (int32 [n, max_blocks] / [n], as block_tables() returned them for
        these seqs) are updated in place with this step's changes."""
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = int(ids.shape[0])
        slots = np.empty(max(n, 1), dtype=np.int64)
        copies = np.empty((max(n, 1), 2), dtype=np.int64)
        nc = _i32(0)
        maxb, tp, cp = 0, None, None
        if tables is not None:
            if (context_lens is None or tables.dtype != np.int32 or context_lens.dtype != np.int32
                    or not tables.flags.c_contiguous or tables.ndim != 2 or tables.shape[0] != n
                    or context_lens.shape != (n,)):
                raise ValueError("tables / context_lens must be C-contiguous int32 [n, max_blocks] / [n]")
            maxb, tp, cp = int(tables.shape[1]), _ptr(tables), _ptr(context_lens)
        st = _lib().pa_bm_append(self._h, _ptr(ids), n, _ptr(slots), _ptr(copies), ctypes.byref(nc),
                                 maxb, tp, cp)
        if st == -2:
            raise ValueError("duplicate sequence ids with tables, or a sequence outgrows max_blocks")
        _check("pa_bm_append", st)
        return slots[:n], copies[:nc.value]

    def append_token(self, seq: int) -> int:
        """Single-token form; copy-on-write pairs accumulate for take_copies()."""
        slots, copies = self.append([seq])
        self.pending_copies.extend((int(a), int(b)) for a, b in copies)
        return int(slots[0])

    def take_copies(self) -> List[Tuple[int, int]]:
        out, self.pending_copies = self.pending_copies, []
        return out

    def shared_prefix(self, seqs: Sequence[int]) -> int:
        """Tokens the sequences share in the same pages, in whole pages
        (pa_decode_shared_prefix's shared_len for a batch of them)."""
        ids = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int64))
        n = int(_lib().pa_bm_shared_prefix(self._h, _ptr(ids) if len(ids) else None, int(ids.shape[0])))
        if n < 0:
            raise KeyError("unknown sequence id")
        return n

    def prefix_groups(self, seqs: Sequence[int]) -> Tuple[np.ndarray, np.ndarray, np.ndarray, int, int]:
        """(group_start [G + 1], group_shared_len [G], seq_shared_len [n],
        max_group_size, max_shared_len): int32 host arrays and the two host
        bounds for pa_decode_shared_prefix_groups on a batch of these
        sequences in this order."""
        ids = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int64))
        n = int(ids.shape[0])
        gs = np.zeros(n + 1, dtype=np.int32)
        gl = np.zeros(max(n, 1), dtype=np.int32)
        sl = np.zeros(max(n, 1), dtype=np.int32)
        bounds = np.zeros(2, dtype=np.int32)
        g = int(_lib().pa_bm_prefix_groups(self._h, _ptr(ids) if n else None, n, _ptr(gs), _ptr(gl), _ptr(sl),
                                           _ptr(bounds[:1]), _ptr(bounds[1:])))
        if g < 0:
            raise KeyError("unknown sequence id")
        return gs[:g + 1], gl[:g], sl[:n], int(bounds[0]), int(bounds[1])

    def block_tables(self, seqs: Sequence[int], max_blocks_per_seq: int,
                     pad_page: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Device-layout inputs: tables [n, max_blocks_per_seq] int32 (pages,
        then pad_page) and context_lens [n] int32."""
        ids = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int64))
        n = int(ids.shape[0])
        tables = np.zeros((max(n, 1), int(max_blocks_per_seq)), dtype=np.int32)
        lens = np.zeros(max(n, 1), dtype=np.int32)
        st = _lib().pa_bm_block_tables(self._h, _ptr(ids), n, int(max_blocks_per_seq), int(pad_page),
                                       _ptr(tables), _ptr(lens))
        if st == -2:
            raise ValueError("a sequence holds more than max_blocks_per_seq pages")
        _check("pa_bm_block_tables", st)
        return tables[:n], lens[:n]
