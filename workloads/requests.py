"""Seeded synthetic request streams for prefix caching: tenants (agents)
whose requests start with the tenant's system prompt and go on with tokens
of their own.  Sizes follow the pages' description of agentic workloads --
shared system prompts, few-shot examples and tool instructions of 5,000 to
20,000 tokens [PagedAttention Internals, "Copy-on-Write and Prefix Sharing"]
-- with token ids drawn uniformly from a 128,256-entry vocabulary (the
Llama-3 tokenizer's size).  Inputs only: no page or cache logic here."""

from __future__ import annotations

from typing import List, Tuple

import numpy as np

VOCAB = 128256


def tenant_requests(num_tenants: int = 8, num_requests: int = 1000, seed: int = 0,
                    system_range=(5000, 20000), suffix_range=(50, 500)) -> List[Tuple[int, List[int]]]:
    """[(tenant, prompt token ids)] in arrival order: tenant drawn uniformly,
    its full system prompt, then a suffix of uniform length in suffix_range."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(system_range[0], system_range[1], size=num_tenants, endpoint=True)
    systems = [rng.integers(0, VOCAB, size=int(n)).tolist() for n in lens]
    out = []
    for _ in range(num_requests):
        t = int(rng.integers(0, num_tenants))
        n = int(rng.integers(suffix_range[0], suffix_range[1], endpoint=True))
        out.append((t, systems[t] + rng.integers(0, VOCAB, size=n).tolist()))
    return out
