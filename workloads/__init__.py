"""Seeded synthetic inputs for paged decode: host block manager plus workload
generators.  Shared by the tests, the benchmark and the smoke check; holds no
attention arithmetic."""

from .blockmgr import BlockManager, OutOfPages  # noqa: F401
from .configs import (  # noqa: F401
    NAMED, Workload, beam_fork, by_name, custom, chunk_elems, copy_probe, llama3_70b,
    llama3_8b, long_context, make_tensors, multi_custom, prefix_share, prompt_chunk, spec_verify, tiny,
    torch_dtype,
)
