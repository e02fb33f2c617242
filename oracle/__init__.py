"""Reference oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct CPU code (numpy, float64) that defines what the
device path must compute.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product library never does,
and nothing here imports the product library.

Pages cited (by title and section, no line numbers):
  [Glossary]  "What is PagedAttention? Definition & Virtual Memory Architecture"
              (esaholic.com AI glossary)
  [Terms]     "Paged Attention" (invest-in.ai AI terminology)
  [Internals] "PagedAttention Internals: How Memory Fragmentation in LLM Serving
              Was Solved" (dailyaiworld.com)

Every function here is pinned by a test that does not reuse its own formula
(closed forms, brute force on tiny inputs, a library attention routine,
invariants, worked examples the pages print).  No function is unpinned.
"""

from .formats import bf16_bits_to_f64, f32_to_bf16_bits, to_f64  # noqa: F401
from .paged_attention import decode, gather_sequence, resolve_slot  # noqa: F401
from .cache_ops import copy_blocks, kv_append  # noqa: F401
from .streaming import online_decode_sequence, segmented_decode_sequence, split_decode_sequence  # noqa: F401
from .prefix_cache import PrefixCachingPool  # noqa: F401
from .multi_query import decode_multi  # noqa: F401
