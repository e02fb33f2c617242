"""KV-cache memory accounting: waste and concurrent capacity, paged vs
contiguous pre-allocation, measured with the native page allocator.

The pages' claims this measures, on the synthetic workloads instead of
production traffic:
  * contiguous pre-allocation reserves each request's maximum length up
    front and wastes most of it; paging wastes only the unfilled tail of each
    sequence's last page [Terms, "Why It Matters in AI" and "Key Points"
    (fragmentation row); Internals, introduction and "The Mathematical Cause
    of KV Cache Fragmentation" item 1 (a 512-token request in a 4,096-token
    reservation wastes 87.5 percent)];
  * one token's KV costs 2 * layers * kv_heads * head_dim * bytes [Internals,
    "The Mathematical Cause of KV Cache Fragmentation"];
  * sequences sharing a prompt store it once [Internals, "Copy-on-Write and
    Prefix Sharing": 100 streams over a 10k-token prompt save over 80
    percent];
  * the same memory therefore serves several times more concurrent requests
    [Internals, introduction and "Benchmark Performance"].

Paged numbers come from an actual allocator: sequences are allocated (and
forked, for shared prompts) in a NativeBlockManager and its free-page count
is read back; capacity admits sequences until the pool reports
out-of-pages.  Contiguous numbers are the reservation arithmetic of a
runtime that reserves `reserve` tokens per request.
"""

from __future__ import annotations

from dataclasses import dataclass, asdict
from typing import Dict, Iterable, List, Optional

import numpy as np

from .block_manager import NativeBlockManager, OutOfPages


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V of one token across all layers."""
    return 2 * int(layers) * int(kv_heads) * int(head_dim) * int(elem_bytes)


@dataclass
class Usage:
    sequences: int
    used_tokens: int          # tokens the sequences attend over (sum of lengths)
    unique_tokens: int        # distinct tokens stored (a shared prompt counts once)
    paged_tokens: int         # page slots the allocator handed out (pages * block_size)
    contiguous_tokens: int    # reservations of a contiguous runtime
    paged_waste: float        # 1 - unique / paged: unfilled slots of held pages
    contiguous_waste: float   # 1 - used / contiguous

    def as_dict(self) -> Dict[str, object]:
        return asdict(self)


def measure_usage(lengths: Iterable[int], block_size: int, reserve: int,
                  prompt: Optional[int] = None) -> Usage:
    """Allocate every sequence in a fresh native manager and read back how
    many page slots it took.  With ``prompt``, all sequences fork one shared
    prompt of that many tokens and append their remaining tokens (lengths
    include the prompt); the paged figure then counts shared pages once."""
    lens = [int(x) for x in lengths]
    need = sum(-(-L // block_size) for L in lens) + 2
    mgr = NativeBlockManager(need, block_size)
    if prompt is None:
        for i, L in enumerate(lens):
            mgr.allocate(i, L)
    else:
        mgr.allocate(-1, prompt)
        for i, L in enumerate(lens):
            if L < prompt:
                raise ValueError("every length must include the shared prompt")
            mgr.fork(-1, i)
            if L > prompt:
                mgr.append(np.full(L - prompt, i, dtype=np.int64))
        mgr.free_sequence(-1)
    pages = need - mgr.num_free()
    used = sum(lens)
    unique = used if prompt is None else prompt + sum(L - prompt for L in lens)
    paged = pages * block_size
    contiguous = len(lens) * int(reserve)
    return Usage(len(lens), used, unique, paged, contiguous,
                 1 - unique / paged if paged else 0.0, 1 - used / contiguous if contiguous else 0.0)


def paged_capacity(budget_tokens: int, block_size: int, lengths: Iterable[int]) -> int:
    """Sequences (taken in the order given, cycling) a pool of budget_tokens
    token slots admits before the allocator runs out of pages."""
    lens = [int(x) for x in lengths]
    mgr = NativeBlockManager(max(int(budget_tokens) // block_size, 1), block_size)
    n = 0
    while True:
        try:
            mgr.allocate(n, lens[n % len(lens)])
        except OutOfPages:
            return n
        n += 1


def contiguous_capacity(budget_tokens: int, reserve: int) -> int:
    """Requests a contiguous runtime fits when each reserves ``reserve`` tokens."""
    return int(budget_tokens) // int(reserve)


def sample_lengths(name: str, n: int, seed: int = 0) -> List[int]:
    """Context lengths drawn like the named workload's (for capacity runs)."""
    rng = np.random.default_rng(seed)
    if name == "llama3_8b":
        return rng.integers(512, 4096, size=n, endpoint=True).tolist()
    if name == "llama3_70b":
        raw = rng.lognormal(mean=np.log(1500.0), sigma=1.0, size=n)
        return np.clip(np.rint(raw), 64, 8192).astype(int).tolist()
    if name == "long_context":
        return [32768] * n
    raise ValueError(name)
