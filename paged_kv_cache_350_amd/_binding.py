"""Thin ctypes binding over libpa.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks that
their dtypes, shapes and devices agree with the C ABI in include/pa.h, and
passes raw device pointers plus the current torch stream to the library.  No
arithmetic of the method happens here; there is no fallback path -- if the
library is missing or the GPU is absent the call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_OK, PA_ERR_NULL, PA_ERR_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = 0, -1, -2, -3, -4, -5
PA_ERR_SCRATCH = -9
STATIC_SCRATCH_BYTES = 32 * 1024 * 1024      # PA_STATIC_SCRATCH_BYTES in include/pa.h
PA_F32, PA_BF16 = 0, 1
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
REUSE = {"auto": 0, "stream": 1, "shared": 2}
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}

_lock = threading.Lock()
_lib_handle: Optional[ctypes.CDLL] = None


class PaError(RuntimeError):
    """A libpa call returned a non-OK status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


_c_int, _c_i64, _c_size, _c_float, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                          ctypes.c_float, ctypes.c_void_p)

_SIGNATURES = {
    "pa_status_string": ([_c_int], ctypes.c_char_p),
    "pa_version": ([], _c_int),
    "pa_decode_partition_size": ([_c_int, _c_int, _c_int, _c_int, _c_int], _c_int),
    "pa_decode_workspace_size": ([_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int], _c_size),
    "pa_kv_append": ([_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _vp], _c_int),
    "pa_decode": ([_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_float, _vp, _vp,
                   _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int, _c_int,
                   _c_int, _vp, _c_size], _c_int),
    "pa_decode_noalloc": ([_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_float, _vp, _vp,
                           _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int, _c_int,
                           _c_int], _c_int),
    "pa_decode_append": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_float, _vp, _vp,
                          _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int, _c_int,
                          _c_int, _vp, _c_size], _c_int),
    "pa_decode_partition": ([_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_float, _vp,
                             _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int, _c_int,
                             _c_int, _vp, _c_size, _vp, _vp, _vp], _c_int),
    "pa_decode_shared_prefix": ([_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_float, _vp, _vp,
                                 _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int, _c_int,
                                 _vp, _c_size, _vp, _vp, _vp], _c_int),
    "pa_decode_shared_prefix_workspace_size": ([_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int],
                                               _c_size),
    "pa_decode_shared_prefix_groups": ([_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_float, _vp, _vp,
                                        _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int,
                                        _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_size, _vp, _vp, _vp],
                                       _c_int),
    "pa_decode_shared_prefix_groups_workspace_size": ([_c_int, _c_int, _c_int, _c_int, _c_int], _c_size),
    "pa_decode_reduce": ([_vp, _c_size, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int],
                         _c_int),
    "pa_copy_blocks": ([_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _vp], _c_int),
    "pa_probe_stream_read": ([_vp, _c_size, _c_int, _c_int, _vp, _vp], _c_int),
    "pa_decode_multi": ([_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, ctypes.c_float, _vp, _vp,
                         _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int,
                         _c_int, _c_int, _vp, _c_size], _c_int),
    "pa_decode_multi_append": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, ctypes.c_float, _vp,
                                _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int,
                                _c_int, _c_int, _vp, _c_size], _c_int),
    "pa_decode_multi_partition_size": ([_c_int, _c_int, _c_int, _c_int, _c_int, _c_int], _c_int),
    "pa_decode_multi_workspace_size": ([_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int],
                                       _c_size),
}


def lib() -> ctypes.CDLL:
    """Load libpa.so (once).  Raises if it has not been built."""
    global _lib_handle
    with _lock:
        if _lib_handle is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"libpa.so not found at {LIB_PATH}; build it with "
                    "`python -m paged_kv_cache_350_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIGNATURES.items():
                fn = getattr(handle, name)
                fn.argtypes = args
                fn.restype = res
            _lib_handle = handle
    return _lib_handle


def status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PaError(fn, status, status_string(status))


def _dev_tensor(name: str, t: torch.Tensor, dtype=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")


def _elem_dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported element type {t.dtype} (float32 or bfloat16)")
    return _DTYPES[t.dtype]


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """(num_blocks, num_kv_heads, head_dim, block_size) from the two cache tensors."""
    _dev_tensor("k_cache", k_cache, ndim=5)
    _dev_tensor("v_cache", v_cache, dtype=k_cache.dtype, ndim=4)
    nb, hkv, nchunk, bs, x = k_cache.shape
    if x * k_cache.element_size() != 16:
        raise ValueError("k_cache innermost axis must span 16 bytes")
    d = nchunk * x
    if tuple(v_cache.shape) != (nb, hkv, d, bs):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} does not match k_cache "
                         f"(expected {(nb, hkv, d, bs)})")
    if k_cache.device != v_cache.device:
        raise ValueError("caches on different devices")
    return nb, hkv, d, bs


def decode_partition_size(num_seqs: int, num_kv_heads: int, max_context_len: int,
                          partition_size: int = 0, reuse: str = "auto") -> int:
    return lib().pa_decode_partition_size(num_seqs, num_kv_heads, max_context_len, partition_size,
                                          REUSE[reuse])


def decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                          max_context_len: int, partition_size: int = 0, reuse: str = "auto") -> int:
    return lib().pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                          max_context_len, partition_size, REUSE[reuse])


def kv_append(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
              k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Scatter new K/V rows [T, Hkv, D] into their slots (in place on the caches)."""
    nb, hkv, d, bs = _cache_dims(k_cache, v_cache)
    _dev_tensor("k", k, dtype=k_cache.dtype, ndim=3)
    _dev_tensor("v", v, dtype=k_cache.dtype, ndim=3)
    _dev_tensor("slot_mapping", slot_mapping, dtype=torch.int64, ndim=1)
    T = k.shape[0]
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d) or slot_mapping.shape[0] != T:
        raise ValueError("k, v, slot_mapping shapes disagree with the caches")
    st = lib().pa_kv_append(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                            k_cache.data_ptr(), v_cache.data_ptr(), T, hkv, d, bs, nb,
                            _elem_dtype(k_cache), _stream(k_cache))
    _check("pa_kv_append", st)


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_mapping: torch.Tensor) -> None:
    """Copy whole pages src -> dst for each row (src, dst) of block_mapping [n, 2]."""
    nb, hkv, d, bs = _cache_dims(k_cache, v_cache)
    _dev_tensor("block_mapping", block_mapping, dtype=torch.int64, ndim=2)
    if block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [n, 2]")
    st = lib().pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), block_mapping.data_ptr(),
                              block_mapping.shape[0], hkv, d, bs, nb, _elem_dtype(k_cache),
                              _stream(k_cache))
    _check("pa_copy_blocks", st)


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len):
    nb, hkv, d, bs = _cache_dims(k_cache, v_cache)
    _dev_tensor("q", q, dtype=k_cache.dtype, ndim=3)
    _dev_tensor("block_tables", block_tables, dtype=torch.int32, ndim=2)
    _dev_tensor("context_lens", context_lens, dtype=torch.int32, ndim=1)
    B, hq, dq = q.shape
    if dq != d:
        raise ValueError(f"q head_dim {dq} != cache head_dim {d}")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens batch size disagrees with q")
    if max_context_len is None:
        raise ValueError("max_context_len (a host-side bound on context_lens) is required")
    return nb, hkv, d, bs, B, hq


def make_workspace(q: torch.Tensor, num_kv_heads: int, max_context_len: int,
                   partition_size: int = 0, reuse: str = "auto"):
    """Allocate the split-path workspace (or None) for a decode call."""
    B, hq, d = q.shape
    n = decode_workspace_size(B, hq, num_kv_heads, d, max_context_len, partition_size, reuse)
    if n == 0:
        return None
    return torch.empty(n // 4, dtype=torch.float32, device=q.device)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           max_context_len: int, out: Optional[torch.Tensor] = None, partition_size: int = 0,
           kernel: str = "auto", workspace: Optional[torch.Tensor] = None,
           reuse: str = "auto") -> torch.Tensor:
    """Paged decode attention; returns out [B, Hq, D] in q's dtype.

    ``reuse`` is "stream" when no page is read by two sequences of the batch,
    "shared" when some are (prefix sharing, beams); it only picks the load
    path."""
    nb, hkv, d, bs, B, hq = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len)
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, dtype=q.dtype, ndim=3)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if workspace is None:
        workspace = make_workspace(q, hkv, max_context_len, partition_size, reuse)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().pa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                         block_tables.data_ptr(), context_lens.data_ptr(), bs, hkv, float(scale),
                         out.data_ptr(), _stream(q), B, hq, d, block_tables.shape[1],
                         int(max_context_len), nb, _elem_dtype(q), int(partition_size),
                         KERNELS[kernel], REUSE[reuse], ws_ptr, ws_bytes)
    _check("pa_decode", st)
    return out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                   max_context_len: int, out: torch.Tensor, partition_size: int = 0,
                   kernel: str = "auto", reuse: str = "auto") -> torch.Tensor:
    """pa_decode without a workspace argument: the split path's partials go to
    the library's static per-GPU scratch (pa_decode_noalloc).  ``out`` must be
    given, so the call allocates nothing; calls on one GPU must not overlap."""
    nb, hkv, d, bs, B, hq = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len)
    _dev_tensor("out", out, dtype=q.dtype, ndim=3)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    st = lib().pa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                 block_tables.data_ptr(), context_lens.data_ptr(), bs, hkv, float(scale),
                                 out.data_ptr(), _stream(q), B, hq, d, block_tables.shape[1],
                                 int(max_context_len), nb, _elem_dtype(q), int(partition_size),
                                 KERNELS[kernel], REUSE[reuse])
    _check("pa_decode_noalloc", st)
    return out


def decode_append(k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                  scale: float, max_context_len: int, slot_mapping: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, partition_size: int = 0, kernel: str = "auto",
                  workspace: Optional[torch.Tensor] = None, reuse: str = "auto") -> torch.Tensor:
    """Append each sequence's newest K/V row [B, Hkv, D] at position L - 1 and
    decode, in one pass; returns out [B, Hq, D].  ``slot_mapping`` [B] int64
    (optional): negative entries mark sequences that append nothing."""
    nb, hkv, d, bs, B, hq = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len)
    _dev_tensor("k_new", k_new, dtype=q.dtype, ndim=3)
    _dev_tensor("v_new", v_new, dtype=q.dtype, ndim=3)
    if tuple(k_new.shape) != (B, hkv, d) or tuple(v_new.shape) != (B, hkv, d):
        raise ValueError("k_new / v_new must be [num_seqs, num_kv_heads, head_dim]")
    sm_ptr = None
    if slot_mapping is not None:
        _dev_tensor("slot_mapping", slot_mapping, dtype=torch.int64, ndim=1)
        if slot_mapping.shape[0] != B:
            raise ValueError("slot_mapping must have one entry per sequence")
        sm_ptr = slot_mapping.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, dtype=q.dtype, ndim=3)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if workspace is None:
        workspace = make_workspace(q, hkv, max_context_len, partition_size, reuse)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().pa_decode_append(k_new.data_ptr(), v_new.data_ptr(), sm_ptr, q.data_ptr(),
                                k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                                context_lens.data_ptr(), bs, hkv, float(scale), out.data_ptr(),
                                _stream(q), B, hq, d, block_tables.shape[1], int(max_context_len), nb,
                                _elem_dtype(q), int(partition_size), KERNELS[kernel], REUSE[reuse],
                                ws_ptr, ws_bytes)
    _check("pa_decode_append", st)
    return out


def _append_args(k_new, v_new, slot_mapping, B: int, hkv: int, d: int, dtype):
    """Pointers for an optional fused append of each sequence's newest rows
    (k_new / v_new [B, Hkv, D], slot_mapping [B] int64 or None); all None
    when no rows are given."""
    if k_new is None and v_new is None:
        return None, None, None
    _dev_tensor("k_new", k_new, dtype=dtype, ndim=3)
    _dev_tensor("v_new", v_new, dtype=dtype, ndim=3)
    if tuple(k_new.shape) != (B, hkv, d) or tuple(v_new.shape) != (B, hkv, d):
        raise ValueError("k_new / v_new must be [num_seqs, num_kv_heads, head_dim]")
    sm = None
    if slot_mapping is not None:
        _dev_tensor("slot_mapping", slot_mapping, dtype=torch.int64, ndim=1)
        if slot_mapping.shape[0] != B:
            raise ValueError("slot_mapping must have one entry per sequence")
        sm = slot_mapping.data_ptr()
    return k_new.data_ptr(), v_new.data_ptr(), sm


def decode_partition(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                     max_context_len: int, partition_size: int, workspace: torch.Tensor,
                     kernel: str = "auto", reuse: str = "auto", k_new=None, v_new=None,
                     slot_mapping=None) -> None:
    """First stage of the split path only (partials into ``workspace``); with
    ``k_new``/``v_new`` [B, Hkv, D] it also does pa_decode_append's append."""
    nb, hkv, d, bs, B, hq = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len)
    _dev_tensor("workspace", workspace, dtype=torch.float32)
    kn, vn, sm = _append_args(k_new, v_new, slot_mapping, B, hkv, d, q.dtype)
    st = lib().pa_decode_partition(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   block_tables.data_ptr(), context_lens.data_ptr(), bs, hkv,
                                   float(scale), _stream(q), B, hq, d, block_tables.shape[1],
                                   int(max_context_len), nb, _elem_dtype(q), int(partition_size),
                                   KERNELS[kernel], REUSE[reuse], workspace.data_ptr(),
                                   workspace.numel() * 4, kn, vn, sm)
    _check("pa_decode_partition", st)


def decode_reduce(workspace: torch.Tensor, context_lens: torch.Tensor, out: torch.Tensor,
                  max_context_len: int, partition_size: int) -> torch.Tensor:
    """Second stage of the split path: merge partials into ``out`` [B, Hq, D]."""
    _dev_tensor("workspace", workspace, dtype=torch.float32)
    _dev_tensor("context_lens", context_lens, dtype=torch.int32, ndim=1)
    _dev_tensor("out", out, ndim=3)
    B, hq, d = out.shape
    st = lib().pa_decode_reduce(workspace.data_ptr(), workspace.numel() * 4, context_lens.data_ptr(),
                                out.data_ptr(), _stream(out), B, hq, d, int(max_context_len),
                                int(partition_size), _elem_dtype(out))
    _check("pa_decode_reduce", st)
    return out


def shared_prefix_len(block_tables, context_lens, block_size: int) -> int:
    """Longest prefix, in whole pages, that every sequence holds in the same
    physical pages: the leading block-table entries equal in all rows, capped
    by the shortest context (host arrays or tensors; host-side bookkeeping
    for pa_decode_shared_prefix, no device work)."""
    import numpy as np
    tables = block_tables.cpu().numpy() if hasattr(block_tables, "cpu") else np.asarray(block_tables)
    lens = context_lens.cpu().numpy() if hasattr(context_lens, "cpu") else np.asarray(context_lens)
    if len(lens) == 0:
        return 0
    same = (tables == tables[:1]).all(axis=0)
    pages = int(np.argmin(same)) if not same.all() else tables.shape[1]
    tokens = min(pages * block_size, int(lens.min()))
    return tokens // block_size * block_size


def shared_prefix_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                 max_context_len: int, shared_len: int, partition_size: int) -> int:
    return lib().pa_decode_shared_prefix_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                        max_context_len, shared_len, partition_size)


def decode_shared_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                         max_context_len: int, shared_len: int, partition_size: int = 0,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, k_new=None, v_new=None,
                         slot_mapping=None) -> torch.Tensor:
    """Decode a batch whose sequences share their first ``shared_len`` tokens
    in the same pages: the shared pages are read once for many sequences'
    queries (see pa_decode_shared_prefix).  With ``k_new`` / ``v_new``
    ([B, Hkv, D]) each sequence's newest rows are appended as by
    decode_append (``slot_mapping`` [B] int64: a negative entry skips)."""
    nb, hkv, d, bs, B, hq = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len)
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, dtype=q.dtype, ndim=3)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if workspace is None:
        n = shared_prefix_workspace_size(B, hq, hkv, d, max_context_len, shared_len, partition_size)
        workspace = torch.empty(max(n, 16) // 4, dtype=torch.float32, device=q.device)
    ws_ptr = workspace.data_ptr()
    ws_bytes = workspace.numel() * workspace.element_size()
    kn, vn, sm = _append_args(k_new, v_new, slot_mapping, B, hkv, d, q.dtype)
    st = lib().pa_decode_shared_prefix(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       block_tables.data_ptr(), context_lens.data_ptr(), bs, hkv,
                                       float(scale), out.data_ptr(), _stream(q), B, hq, d,
                                       block_tables.shape[1], int(max_context_len), nb, _elem_dtype(q),
                                       int(shared_len), int(partition_size), ws_ptr, ws_bytes, kn, vn, sm)
    _check("pa_decode_shared_prefix", st)
    return out


def decode_shared_prefix_groups(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                                max_context_len: int, group_start: torch.Tensor, group_shared_len: torch.Tensor,
                                seq_shared_len: torch.Tensor, max_group_size: int, max_shared_len: int,
                                partition_size: int = 0, out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None, k_new=None, v_new=None,
                                slot_mapping=None) -> torch.Tensor:
    """Decode a batch of groups of sequences, each group sharing its own
    prefix pages (see pa_decode_shared_prefix_groups); the group arrays are
    int32 device tensors."""
    nb, hkv, d, bs, B, hq = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len)
    G = int(group_shared_len.shape[0])
    _dev_tensor("group_start", group_start, dtype=torch.int32, ndim=1)
    _dev_tensor("group_shared_len", group_shared_len, dtype=torch.int32, ndim=1)
    _dev_tensor("seq_shared_len", seq_shared_len, dtype=torch.int32, ndim=1)
    if group_start.shape[0] != G + 1 or seq_shared_len.shape[0] != B:
        raise ValueError("group_start must have num_groups + 1 entries, seq_shared_len num_seqs")
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, dtype=q.dtype, ndim=3)
    if workspace is None:
        n = lib().pa_decode_shared_prefix_groups_workspace_size(B, hq, d, int(max_context_len),
                                                                int(partition_size))
        workspace = torch.empty(max(n, 16) // 4, dtype=torch.float32, device=q.device)
    kn, vn, sm = _append_args(k_new, v_new, slot_mapping, B, hkv, d, q.dtype)
    st = lib().pa_decode_shared_prefix_groups(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        bs, hkv, float(scale), out.data_ptr(), _stream(q), B, hq, d, block_tables.shape[1],
        int(max_context_len), nb, _elem_dtype(q), G, group_start.data_ptr(), group_shared_len.data_ptr(),
        seq_shared_len.data_ptr(), int(max_group_size), int(max_shared_len), int(partition_size),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), kn, vn, sm)
    _check("pa_decode_shared_prefix_groups", st)
    return out


def decode_multi_partition_size(num_seqs: int, num_heads: int, num_kv_heads: int, max_context_len: int,
                                max_query_len: int, partition_size: int = 0) -> int:
    return lib().pa_decode_multi_partition_size(num_seqs, num_heads, num_kv_heads, max_context_len,
                                                max_query_len, partition_size)


def decode_multi_workspace_size(num_seqs: int, num_tokens: int, num_heads: int, num_kv_heads: int,
                                head_dim: int, max_context_len: int, max_query_len: int,
                                partition_size: int = 0) -> int:
    return lib().pa_decode_multi_workspace_size(num_seqs, num_tokens, num_heads, num_kv_heads, head_dim,
                                                max_context_len, max_query_len, partition_size)


def decode_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
                 scale: float, max_context_len: int, max_query_len: int,
                 out: Optional[torch.Tensor] = None, partition_size: int = 0,
                 workspace: Optional[torch.Tensor] = None, reuse: str = "auto",
                 k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention for several new tokens per sequence: q [T, Hq, D] packed by
    sequence, query_start [B + 1] int32; row query_start[b] + j attends
    causally over positions 0 .. L_b - n_b + j.  Without k_new / v_new the
    new tokens' rows must already be in the caches; with them ([T, Hkv, D],
    aligned with q) the same launch appends them (pa_decode_multi_append).
    Returns out [T, Hq, D]."""
    nb, hkv, d, bs = _cache_dims(k_cache, v_cache)
    _dev_tensor("q", q, dtype=k_cache.dtype, ndim=3)
    _dev_tensor("block_tables", block_tables, dtype=torch.int32, ndim=2)
    _dev_tensor("context_lens", context_lens, dtype=torch.int32, ndim=1)
    _dev_tensor("query_start", query_start, dtype=torch.int32, ndim=1)
    T, hq, dq = q.shape
    B = context_lens.shape[0]
    if dq != d:
        raise ValueError(f"q head_dim {dq} != cache head_dim {d}")
    if block_tables.shape[0] != B or query_start.shape[0] != B + 1:
        raise ValueError("block_tables / query_start disagree with context_lens")
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor("out", out, dtype=q.dtype, ndim=3)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if workspace is None:
        n = decode_multi_workspace_size(B, T, hq, hkv, d, max_context_len, max_query_len, partition_size)
        workspace = torch.empty(n // 4, dtype=torch.float32, device=q.device) if n else None
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
            context_lens.data_ptr(), query_start.data_ptr(), bs, hkv, float(scale), out.data_ptr(), _stream(q),
            B, T, hq, d, block_tables.shape[1], int(max_context_len), int(max_query_len), nb, _elem_dtype(q),
            int(partition_size), REUSE[reuse], ws_ptr, ws_bytes)
    if k_new is None and v_new is None:
        _check("pa_decode_multi", lib().pa_decode_multi(*args))
        return out
    _dev_tensor("k_new", k_new, dtype=q.dtype, ndim=3)
    _dev_tensor("v_new", v_new, dtype=q.dtype, ndim=3)
    if tuple(k_new.shape) != (T, hkv, d) or tuple(v_new.shape) != (T, hkv, d):
        raise ValueError("k_new / v_new must be [num_tokens, num_kv_heads, head_dim], aligned with q")
    _check("pa_decode_multi_append", lib().pa_decode_multi_append(k_new.data_ptr(), v_new.data_ptr(), *args))
    return out


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, nontemporal: bool = True,
                      num_workgroups: int = 0) -> None:
    """Read every byte of ``buf`` once (measurement helper, not the decode path)."""
    _dev_tensor("buf", buf)
    _dev_tensor("sink", sink, dtype=torch.int32)
    st = lib().pa_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                    int(bool(nontemporal)), int(num_workgroups), sink.data_ptr(),
                                    _stream(buf))
    _check("pa_probe_stream_read", st)
