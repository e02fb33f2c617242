"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute lives in libpa.so (hand-written HIP kernels behind the C ABI in
include/pa.h); this package is the thin Python binding that tests and the
benchmark call.  Build the library with
``python -m paged_kv_cache_350_amd.build``.
"""

from ._binding import (  # noqa: F401
    KERNELS, LIB_PATH, REUSE, PA_BF16, PA_ERR_ARG, PA_ERR_HIP, PA_ERR_NULL, PA_ERR_UNSUPPORTED,
    PA_ERR_SCRATCH, PA_ERR_WORKSPACE, PA_F32, PA_OK, STATIC_SCRATCH_BYTES, PaError, copy_blocks, decode,
    decode_append, decode_noalloc, decode_partition,
    decode_multi, decode_multi_partition_size, decode_multi_workspace_size,
    decode_partition_size, decode_reduce, decode_shared_prefix, decode_shared_prefix_groups,
    decode_workspace_size, kv_append, lib,
    shared_prefix_len, shared_prefix_workspace_size,
    make_workspace, probe_stream_read, status_string,
)
from .block_manager import NativeBlockManager, OutOfPages  # noqa: F401,E402
