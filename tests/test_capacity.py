"""KV waste and capacity accounting (CPU only): the native allocator's
measurements against closed forms written out here, and the worked numbers
the pages print (tests/golden/*.json)."""

import json
import math
import os

import numpy as np
import pytest

import workloads

pa = pytest.importorskip("paged_kv_cache_350_amd")
from paged_kv_cache_350_amd import capacity as C  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_bytes_per_token_matches_the_pages():
    ex = load("kv_bytes_llama3_70b.json")
    assert C.kv_bytes_per_token(ex["layers"], ex["kv_heads"], ex["head_dim"],
                                ex["bytes_per_element"]) == ex["bytes_per_token"]


def test_internal_fragmentation_example():
    ex = load("internal_fragmentation.json")
    u = C.measure_usage([ex["used_tokens"]], 16, ex["reserved_tokens"])
    assert u.contiguous_waste == ex["waste_fraction"]
    assert u.paged_waste == 0.0                    # 512 tokens fill 32 pages exactly
    u = C.measure_usage([ex["used_tokens"] + 1], 16, ex["reserved_tokens"])
    assert u.paged_tokens == 33 * 16               # one more token: one more page, 15 slots idle


@pytest.mark.parametrize("name", ["llama3_8b", "llama3_70b", "long_context", "tiny"])
def test_paged_usage_is_the_page_rounding(name):
    w = workloads.by_name(name)
    bs = w.block_size
    u = C.measure_usage(w.context_lens, bs, 8192)
    held = sum(math.ceil(int(L) / bs) * bs for L in w.context_lens)
    assert u.paged_tokens == held
    assert u.used_tokens == u.unique_tokens == int(w.context_lens.sum())
    assert math.isclose(u.paged_waste, 1 - u.used_tokens / held)
    assert math.isclose(u.contiguous_waste, 1 - u.used_tokens / (8192 * w.num_seqs))


def test_prefix_sharing_saving():
    """100 streams over one 10,000-token prompt (block 32): the prompt is
    stored once; each stream with its own tokens copies the partly filled
    last prompt page and adds pages for its suffix."""
    w = workloads.prefix_share()
    bs, prompt = w.block_size, 10000
    u = C.measure_usage(w.context_lens, bs, 10512, prompt=prompt)
    shared = math.ceil(prompt / bs)
    full = prompt // bs
    private = sum(math.ceil(int(L) / bs) - full for L in w.context_lens if int(L) > prompt)
    assert u.paged_tokens == (shared + private) * bs
    flat = C.measure_usage(w.context_lens, bs, 10512)
    saving = 1 - u.paged_tokens / flat.paged_tokens
    assert saving > 0.80                           # the pages: "over 80 percent"
    assert u.unique_tokens == prompt + int(w.context_lens.sum()) - prompt * w.num_seqs


def test_capacity_closed_forms():
    lens = C.sample_lengths("llama3_70b", 512, seed=3)
    budget = 200_000
    n = C.paged_capacity(budget, 16, lens)
    pages, want = budget // 16, 0
    for L in lens * 4:
        pages -= math.ceil(L / 16)
        if pages < 0:
            break
        want += 1
    assert n == want
    assert C.contiguous_capacity(budget, 8192) == budget // 8192
    assert n > 3 * C.contiguous_capacity(budget, 8192)   # log-normal lengths vs max-length reservations
