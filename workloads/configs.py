"""Seeded synthetic decode workloads.

Every workload is one decode step of one attention layer: each sequence has a
context of ``L`` tokens in a paged KV cache, the newest token's K/V row is
appended into its slot, then one query per sequence attends over all ``L``
tokens.  This module only *builds inputs*: lengths, page assignments,
copy-on-write copies, slots and random values.  It holds none of the
attention arithmetic, and both the oracle side and the device side consume
what it produces.

Host structure (lengths, page permutation, tables) is drawn with numpy's
``default_rng(seed)`` in a fixed order: context lengths first, then the
permutation of physical page ids.  Pages are handed out by the FIFO block
manager in permutation order, so sequence ``b`` gets the next pages of the
permuted pool.  Values (Q, K, V, new rows) are N(0, 1) drawn with a seeded
``torch.Generator`` on the target device and rounded once to the storage
dtype (round-to-nearest-even); the oracle always reads back the exact bytes
that were produced, so no value is ever regenerated on another device.

Every slot that does not hold a token before the step (spare pages, the tail
of partly filled pages, the slots about to be appended, the padding page that
fills unused block-table entries) is filled with NaN, so a stray read of any
of them shows up in the output.

Device layouts (the pages fix none; these are this library's choices):
  q, out     [num_seqs][num_heads][head_dim]
  k_new/v_new[num_tokens][num_kv_heads][head_dim]
  k_cache    [num_blocks][num_kv_heads][head_dim // X][block_size][X],
             X = 16 bytes / element size (8 for bf16, 4 for fp32)
  v_cache    [num_blocks][num_kv_heads][head_dim][block_size]
  block_tables [num_seqs][max_blocks_per_seq] int32, context_lens [num_seqs] int32
  slot_mapping [num_tokens] int64, copy_pairs [n][2] int64 (src, dst)
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .blockmgr import BlockManager

PROMPT_SEQ = -1      # sequence id of a shared prompt before it is forked


def _manager(factory, num_blocks: int, block_size: int, free_order):
    """Block manager for a workload: the host fixture, or any class with the
    same interface passed as ``factory`` (e.g. the native one)."""
    return (factory or BlockManager)(num_blocks, block_size, free_order=free_order)

ELEM_BYTES = {"f32": 4, "bf16": 2}


def chunk_elems(dtype: str) -> int:
    """Elements per 16-byte chunk of a K row (the innermost K-cache axis)."""
    return 16 // ELEM_BYTES[dtype]


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray          # int32 [B], length after this step's appends
    block_tables: np.ndarray          # int32 [B, max_blocks_per_seq]
    pad_page: int                     # NaN page used for unused table entries
    resident: np.ndarray              # bool [num_blocks, block_size]: holds a token before the step
    copy_pairs: np.ndarray            # int64 [n, 2]
    append_slots: np.ndarray          # int64 [T]
    append_seq: np.ndarray            # int32 [T] sequence each appended token belongs to
    partition_size: int = 0           # 0 = library default
    description: str = ""
    extra: Dict[str, object] = field(default_factory=dict)
    query_lens: Optional[np.ndarray] = None   # int32 [B]: new tokens per sequence (multi-query); None = 1 query each

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def query_start(self) -> Optional[np.ndarray]:
        """int32 [B + 1] offsets of each sequence's query rows (multi-query only)."""
        if self.query_lens is None:
            return None
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        return 1 if self.query_lens is None else max(int(self.query_lens.max()), 1)

    @property
    def scale(self) -> float:
        """1/sqrt(head_dim), as the fp32 value handed to the device."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def x(self) -> int:
        return chunk_elems(self.dtype)

    def k_cache_shape(self) -> Tuple[int, ...]:
        return (self.num_blocks, self.num_kv_heads, self.head_dim // self.x,
                self.block_size, self.x)

    def v_cache_shape(self) -> Tuple[int, ...]:
        return (self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size)

    def kv_bytes_per_token(self) -> int:
        """K+V bytes one token occupies in one layer (2 * Hkv * D * elem)."""
        return 2 * self.num_kv_heads * self.head_dim * self.elem_bytes

    def algorithmic_kv_bytes(self) -> int:
        """K/V bytes one decode step must read: every context token once per kv head."""
        return int(self.context_lens.astype(np.int64).sum()) * self.kv_bytes_per_token()

    def multi_flops(self) -> int:
        """Multiply-adds x 2 of the attention a multi-query step computes: each
        query row j of a sequence with n new tokens sees L - n + j + 1
        positions, and costs 2 D flops per position for Q.K^T and 2 D for
        P.V, for every query head."""
        total = 0
        news = np.ones(self.num_seqs, dtype=np.int64) if self.query_lens is None else self.query_lens
        for L, n in zip(self.context_lens.astype(np.int64), np.asarray(news, dtype=np.int64)):
            n = min(int(n), int(L))
            total += n * (int(L) - n) + n * (n + 1) // 2
        return 4 * self.head_dim * self.num_heads * total

    def unique_kv_bytes(self) -> int:
        """Bytes of distinct (page, offset) slots read, for shared-page workloads."""
        bs = self.block_size
        seen = np.zeros((self.num_blocks, bs), dtype=bool)
        for b in range(self.num_seqs):
            L = int(self.context_lens[b])
            if L == 0:
                continue
            pos = np.arange(L)
            seen[self.block_tables[b, pos // bs], pos % bs] = True
        return int(seen.sum()) * self.kv_bytes_per_token()

    def summary(self) -> Dict[str, object]:
        return {
            "workload": self.name, "seed": self.seed, "dtype": self.dtype,
            "num_seqs": self.num_seqs, "num_heads": self.num_heads,
            "num_kv_heads": self.num_kv_heads, "head_dim": self.head_dim,
            "block_size": self.block_size, "num_blocks": self.num_blocks,
            "sum_context": int(self.context_lens.astype(np.int64).sum()),
            "max_context_len": self.max_context_len,
        }


# ---------------------------------------------------------------------------
# host structure
# ---------------------------------------------------------------------------

def _tables_from(mgr: BlockManager, seqs: Sequence, pad_page: int) -> np.ndarray:
    width = max([len(mgr.tables[s]) for s in seqs] + [1])
    out = np.full((len(seqs), width), pad_page, dtype=np.int32)
    for i, s in enumerate(seqs):
        t = mgr.tables[s]
        out[i, :len(t)] = t
    return out


def _resident_mask(num_blocks: int, bs: int, tables: List[List[int]],
                   lengths: Sequence[int]) -> np.ndarray:
    res = np.zeros((num_blocks, bs), dtype=bool)
    for t, L in zip(tables, lengths):
        L = int(L)
        if L == 0:
            continue
        pos = np.arange(L)
        res[np.asarray(t, dtype=np.int64)[pos // bs], pos % bs] = True
    return res


def _plain(name: str, seed: int, dtype: str, lens: np.ndarray, num_heads: int,
           num_kv_heads: int, head_dim: int, block_size: int,
           rng: np.random.Generator, num_blocks: Optional[int] = None,
           partition_size: int = 0, description: str = "",
           first_table: Optional[Sequence[int]] = None, manager=None) -> Workload:
    """Independent sequences; each appends its newest token (position L-1).

    Before the step every sequence holds L-1 tokens; the block manager gives
    it pages for those, then the step's append may open one more page.
    """
    lens = np.asarray(lens, dtype=np.int64)
    if (lens < 1).any():
        raise ValueError("every sequence needs at least the token being appended")
    bs = block_size
    need = int(sum(-(-int(L) // bs) for L in lens))
    if num_blocks is None:
        num_blocks = int(math.ceil(1.1 * need))
        if num_blocks <= need:
            num_blocks = need + 1           # always keep one spare page for padding
    perm = rng.permutation(num_blocks)
    if first_table is not None:
        # A fixed page list for sequence 0 (worked example from the pages):
        # move those ids to the front of the free list, keep the rest in order.
        first = [int(x) for x in first_table]
        rest = [int(x) for x in perm if int(x) not in first]
        perm = np.asarray(first + rest)
    mgr = _manager(manager, num_blocks, bs, perm)
    seqs = list(range(len(lens)))
    for b in seqs:
        mgr.allocate(b, int(lens[b]) - 1)
    pre_tables = [list(mgr.tables[b]) for b in seqs]
    slots = np.array([mgr.append_token(b) for b in seqs], dtype=np.int64)
    if mgr.pending_copies:
        raise AssertionError("independent sequences never share pages")
    if mgr.num_free() == 0:
        raise ValueError("pool has no spare page for padding")
    pad_page = int(mgr.free[-1])
    tables = _tables_from(mgr, seqs, pad_page)
    resident = _resident_mask(num_blocks, bs, pre_tables, lens - 1)
    return Workload(
        name=name, seed=seed, dtype=dtype, num_heads=num_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs,
        num_blocks=num_blocks, context_lens=lens.astype(np.int32),
        block_tables=tables, pad_page=pad_page, resident=resident,
        copy_pairs=np.zeros((0, 2), dtype=np.int64), append_slots=slots,
        append_seq=np.arange(len(lens), dtype=np.int32),
        partition_size=partition_size, description=description)


def tiny(seed: int = 0, figure_table: bool = False, manager=None) -> Workload:
    """2 sequences of 36 and 42 tokens, block 16, pool of 16 pages, 4 q = 4 kv
    heads, head_dim 64, fp32.  With ``figure_table`` sequence 0 sits on pages
    7, 14, 2 as in the page-table figure of "What is PagedAttention?"."""
    rng = np.random.default_rng(seed)
    lens = np.array([36, 42])
    return _plain("tiny" + ("_figure" if figure_table else ""), seed, "f32", lens,
                  4, 4, 64, 16, rng, num_blocks=16,
                  first_table=[7, 14, 2] if figure_table else None, manager=manager,
                  description="2 seqs (36, 42 tokens), bs 16, pool 16, 4/4 heads, D 64, fp32")


def llama3_8b(seed: int = 1, num_seqs: int = 64, len_range: Tuple[int, int] = (512, 4096),
              dtype: str = "bf16", block_size: int = 16, partition_size: int = 0,
              manager=None) -> Workload:
    """Llama-3-8B-shaped layer: 32 q / 8 kv heads, head_dim 128, block 16,
    context lengths integer-uniform in ``len_range`` (inclusive), pool = pages
    needed + 10 %, ids randomly permuted."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_range[0], len_range[1], size=num_seqs, endpoint=True)
    return _plain("llama3_8b" if (num_seqs, len_range) == (64, (512, 4096)) else
                  f"llama3_8b_b{num_seqs}_l{len_range[0]}-{len_range[1]}",
                  seed, dtype, lens, 32, 8, 128, block_size, rng,
                  partition_size=partition_size, manager=manager,
                  description=f"{num_seqs} seqs, L~U[{len_range[0]},{len_range[1]}], "
                              f"32/8 heads, D 128, bs {block_size}, {dtype}")


def llama3_70b(seed: int = 2, num_seqs: int = 256, median: float = 1500.0,
               sigma: float = 1.0, clip: Tuple[int, int] = (64, 8192),
               dtype: str = "bf16", partition_size: int = 0, manager=None) -> Workload:
    """Llama-3-70B-shaped layer: 64 q / 8 kv heads, head_dim 128, block 16,
    context lengths round(LogNormal(ln median, sigma)) clipped to ``clip``."""
    rng = np.random.default_rng(seed)
    raw = rng.lognormal(mean=math.log(median), sigma=sigma, size=num_seqs)
    lens = np.clip(np.rint(raw), clip[0], clip[1]).astype(np.int64)
    return _plain("llama3_70b" if num_seqs == 256 and clip == (64, 8192) else
                  f"llama3_70b_b{num_seqs}_clip{clip[0]}-{clip[1]}",
                  seed, dtype, lens, 64, 8, 128, 16, rng,
                  partition_size=partition_size, manager=manager,
                  description=f"{num_seqs} seqs, L=clip(round(LogNormal(ln {median:g}, {sigma:g})), "
                              f"{clip[0]}, {clip[1]}), 64/8 heads, D 128, bs 16, {dtype}")


def long_context(seed: int = 4, num_seqs: int = 8, context: int = 32768,
                 partition_size: int = 512, manager=None) -> Workload:
    """Long-context split path: ``num_seqs`` x ``context`` tokens, 32 q / 8 kv
    heads, head_dim 128, block 16, bf16, partitions of 512 tokens."""
    rng = np.random.default_rng(seed)
    lens = np.full(num_seqs, context, dtype=np.int64)
    return _plain("long_context" if (num_seqs, context) == (8, 32768) else
                  f"long_context_b{num_seqs}_l{context}",
                  seed, "bf16", lens, 32, 8, 128, 16, rng,
                  partition_size=partition_size, manager=manager,
                  description=f"{num_seqs} x {context} tokens, 32/8 heads, D 128, bs 16, bf16, "
                              f"partition {partition_size}")


def prefix_share(seed: int = 3, num_seqs: int = 100, prefix: int = 10000,
                 suffix_max: int = 512, manager=None) -> Workload:
    """Shared system prompt: ``num_seqs`` sequences fork one ``prefix``-token
    prompt, then each appends its own suffix of U{0..suffix_max} tokens.
    Writing into the partly filled shared page triggers copy-on-write.
    32 q / 8 kv heads, head_dim 128, block 32, bf16."""
    rng = np.random.default_rng(seed)
    bs = 32
    suffix = rng.integers(0, suffix_max, size=num_seqs, endpoint=True)
    lens = prefix + suffix
    shared = -(-prefix // bs)
    private = 0
    for L in lens:                 # worst case: every sequence copies the shared tail page
        private += -(-int(L) // bs) - (prefix // bs)
    need = shared + private
    num_blocks = int(math.ceil(1.1 * need))
    perm = rng.permutation(num_blocks)
    mgr = _manager(manager, num_blocks, bs, perm)
    mgr.allocate(PROMPT_SEQ, prefix)
    prompt_pages = list(mgr.tables[PROMPT_SEQ])
    for b in range(num_seqs):
        mgr.fork(PROMPT_SEQ, b)
    mgr.free_sequence(PROMPT_SEQ)
    resident = _resident_mask(num_blocks, bs, [prompt_pages], [prefix])
    slots, owner = [], []
    for b in range(num_seqs):
        for _ in range(int(suffix[b])):
            slots.append(mgr.append_token(b))
            owner.append(b)
    copies = mgr.take_copies()
    pad_page = int(mgr.free[-1])
    tables = _tables_from(mgr, list(range(num_seqs)), pad_page)
    w = Workload(
        name="prefix_share" if (num_seqs, prefix, suffix_max) == (100, 10000, 512) else
        f"prefix_share_b{num_seqs}_p{prefix}_s{suffix_max}",
        seed=seed, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
        block_size=bs, num_blocks=num_blocks, context_lens=lens.astype(np.int32),
        block_tables=tables, pad_page=pad_page, resident=resident,
        copy_pairs=np.asarray(copies, dtype=np.int64).reshape(-1, 2),
        append_slots=np.asarray(slots, dtype=np.int64),
        append_seq=np.asarray(owner, dtype=np.int32),
        description=f"{num_seqs} seqs share a {prefix}-token prefix + U{{0..{suffix_max}}} "
                    f"suffix, 32/8 heads, D 128, bs 32, bf16")
    w.extra["shared_pages"] = prompt_pages
    return w


def prefix_groups(seed: int = 5, num_groups: int = 4, group_size: int = 25, prompt: int = 4096,
                  suffix_max: int = 512, manager=None) -> Workload:
    """Several tenants' prompts at once: ``num_groups`` prompts of ``prompt``
    tokens, each forked to ``group_size`` sequences (consecutive ids) that
    append their own suffixes of U{0..suffix_max} tokens.  32 q / 8 kv heads,
    head_dim 128, block 32, bf16.  extra["groups"] lists (first sequence,
    size) per group."""
    rng = np.random.default_rng(seed)
    bs = 32
    num_seqs = num_groups * group_size
    suffix = rng.integers(0, suffix_max, size=num_seqs, endpoint=True)
    lens = prompt + suffix
    need = num_groups * -(-prompt // bs)
    for L in lens:
        need += -(-int(L) // bs) - (prompt // bs)
    num_blocks = int(math.ceil(1.1 * need))
    perm = rng.permutation(num_blocks)
    mgr = _manager(manager, num_blocks, bs, perm)
    prompt_tables, groups = [], []
    for gi in range(num_groups):
        pid = PROMPT_SEQ - gi
        mgr.allocate(pid, prompt)
        prompt_tables.append(list(mgr.tables[pid]))
        for b in range(gi * group_size, (gi + 1) * group_size):
            mgr.fork(pid, b)
        mgr.free_sequence(pid)
        groups.append((gi * group_size, group_size))
    resident = _resident_mask(num_blocks, bs, prompt_tables, [prompt] * num_groups)
    slots, owner = [], []
    for b in range(num_seqs):
        for _ in range(int(suffix[b])):
            slots.append(mgr.append_token(b))
            owner.append(b)
    copies = mgr.take_copies()
    pad_page = int(mgr.free[-1])
    tables = _tables_from(mgr, list(range(num_seqs)), pad_page)
    w = Workload(
        name="prefix_groups" if (num_groups, group_size, prompt, suffix_max) == (4, 25, 4096, 512) else
        f"prefix_groups_g{num_groups}x{group_size}_p{prompt}_s{suffix_max}",
        seed=seed, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
        block_size=bs, num_blocks=num_blocks, context_lens=lens.astype(np.int32),
        block_tables=tables, pad_page=pad_page, resident=resident,
        copy_pairs=np.asarray(copies, dtype=np.int64).reshape(-1, 2),
        append_slots=np.asarray(slots, dtype=np.int64),
        append_seq=np.asarray(owner, dtype=np.int32),
        description=f"{num_groups} prompts of {prompt} tokens x {group_size} sequences each + U{{0..{suffix_max}}} "
                    f"suffix, 32/8 heads, D 128, bs 32, bf16")
    w.extra["shared_pages"] = [p for t in prompt_tables for p in t]
    w.extra["groups"] = groups
    return w


def beam_fork(seed: int = 3, beams: int = 8, prompt: int = 32768, shared_gen: int = 5,
              manager=None) -> Workload:
    """Beam search over one long prompt: the prompt plus ``shared_gen``
    generated tokens are shared by ``beams`` beams; each beam then appends its
    own token, so every beam but the last holder copies the shared tail page.
    32 q / 8 kv heads, head_dim 128, block 32, bf16."""
    rng = np.random.default_rng(seed + 1000)
    bs = 32
    base = prompt + shared_gen
    shared = -(-base // bs)
    need = shared + (beams - 1)
    num_blocks = int(math.ceil(1.1 * need))
    perm = rng.permutation(num_blocks)
    mgr = _manager(manager, num_blocks, bs, perm)
    mgr.allocate(0, prompt)
    for _ in range(shared_gen):
        mgr.append_token(0)
    shared_pages = list(mgr.tables[0])
    for b in range(1, beams):
        mgr.fork(0, b)
    resident = _resident_mask(num_blocks, bs, [shared_pages], [base])
    slots = np.array([mgr.append_token(b) for b in range(beams)], dtype=np.int64)
    copies = mgr.take_copies()
    pad_page = int(mgr.free[-1])
    tables = _tables_from(mgr, list(range(beams)), pad_page)
    lens = np.full(beams, base + 1, dtype=np.int32)
    w = Workload(
        name="beam_fork" if (beams, prompt, shared_gen) == (8, 32768, 5) else
        f"beam_fork_k{beams}_p{prompt}",
        seed=seed, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
        block_size=bs, num_blocks=num_blocks, context_lens=lens, block_tables=tables,
        pad_page=pad_page, resident=resident,
        copy_pairs=np.asarray(copies, dtype=np.int64).reshape(-1, 2),
        append_slots=slots, append_seq=np.arange(beams, dtype=np.int32),
        description=f"{beams} beams fork a {prompt}-token prompt after {shared_gen} shared "
                    f"tokens, 32/8 heads, D 128, bs 32, bf16")
    w.extra["shared_pages"] = shared_pages
    return w


def _multi(name: str, seed: int, lens, news, num_heads: int, num_kv_heads: int, head_dim: int,
           block_size: int, rng: np.random.Generator, description: str, manager=None) -> Workload:
    """Independent sequences that each bring n_b new tokens at once: before
    the step sequence b holds L_b - n_b tokens, the step appends n_b (slots
    in position order, pages opened as blocks fill), then n_b queries attend
    (multi-query).  Pool = pages needed + 10 %, ids randomly permuted, bf16."""
    lens = np.asarray(lens, dtype=np.int64)
    news = np.asarray(news, dtype=np.int64)
    if (news < 0).any() or (news > lens).any():
        raise ValueError("0 <= new tokens <= context length")
    bs = block_size
    need = int(sum(-(-int(L) // bs) for L in lens))
    num_blocks = max(int(math.ceil(1.1 * need)), need + 1)
    perm = rng.permutation(num_blocks)
    mgr = _manager(manager, num_blocks, bs, perm)
    seqs = list(range(len(lens)))
    for b in seqs:
        mgr.allocate(b, int(lens[b] - news[b]))
    pre_tables = [list(mgr.tables[b]) for b in seqs]
    slots, owner = [], []
    for b in seqs:
        for _ in range(int(news[b])):
            slots.append(mgr.append_token(b))
            owner.append(b)
    pad_page = int(mgr.free[-1])
    return Workload(
        name=name, seed=seed, dtype="bf16", num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=bs, num_blocks=num_blocks,
        context_lens=lens.astype(np.int32), block_tables=_tables_from(mgr, seqs, pad_page),
        pad_page=pad_page, resident=_resident_mask(num_blocks, bs, pre_tables, lens - news),
        copy_pairs=np.zeros((0, 2), dtype=np.int64), append_slots=np.asarray(slots, dtype=np.int64),
        append_seq=np.asarray(owner, dtype=np.int32), description=description,
        query_lens=news.astype(np.int32))


def spec_verify(seed: int = 5, num_seqs: int = 64, len_range: Tuple[int, int] = (512, 4096),
                drafts: int = 4, manager=None) -> Workload:
    """Speculative-decoding verification on the Llama-3-8B-shaped batch:
    every sequence scores its last accepted token plus ``drafts`` draft
    tokens (n = drafts + 1 queries), context lengths (new tokens included)
    integer-uniform in ``len_range``; 32 q / 8 kv heads, head_dim 128,
    block 16, bf16."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_range[0], len_range[1], size=num_seqs, endpoint=True)
    news = np.full(num_seqs, drafts + 1)
    return _multi("spec_verify" if (num_seqs, len_range, drafts) == (64, (512, 4096), 4) else
                  f"spec_verify_b{num_seqs}_l{len_range[0]}-{len_range[1]}_k{drafts}",
                  seed, lens, news, 32, 8, 128, 16, rng, manager=manager,
                  description=f"{num_seqs} seqs, L~U[{len_range[0]},{len_range[1]}], {drafts + 1} queries "
                              f"each (verify {drafts} drafts), 32/8 heads, D 128, bs 16, bf16")


def prompt_chunk(seed: int = 6, num_seqs: int = 8, context: int = 4096, chunk: int = 512,
                 manager=None) -> Workload:
    """Chunked prefill on the Llama-3-8B-shaped heads: every sequence holds
    ``context - chunk`` tokens and appends the next ``chunk`` tokens of its
    prompt, whose queries attend causally (n = chunk queries each); 32 q / 8
    kv heads, head_dim 128, block 16, bf16."""
    rng = np.random.default_rng(seed)
    lens = np.full(num_seqs, context)
    news = np.full(num_seqs, chunk)
    return _multi("prompt_chunk" if (num_seqs, context, chunk) == (8, 4096, 512) else
                  f"prompt_chunk_b{num_seqs}_l{context}_c{chunk}",
                  seed, lens, news, 32, 8, 128, 16, rng, manager=manager,
                  description=f"{num_seqs} seqs x {chunk} prompt tokens over {context - chunk} cached "
                              f"(chunked prefill), 32/8 heads, D 128, bs 16, bf16")


def multi_custom(name: str, seed: int, lens, news, num_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, manager=None) -> Workload:
    """Multi-query sequences with explicit context lengths and new-token counts."""
    rng = np.random.default_rng(seed)
    return _multi(name, seed, lens, news, num_heads, num_kv_heads, head_dim, block_size, rng,
                  manager=manager, description=f"{len(lens)} seqs, {num_heads}/{num_kv_heads} heads, "
                                               f"D {head_dim}, bs {block_size}, bf16, multi-query")


def copy_probe(beams: int = 8, prompt: int = 32768) -> np.ndarray:
    """Eager fork of a ``prompt``-token prompt (block 32) to ``beams-1`` beams:
    the page copies copy-on-write avoids.  Returns (src, dst) pairs over a pool
    of ``beams * prompt / 32`` pages."""
    pages = prompt // 32
    src = np.tile(np.arange(pages), beams - 1)
    dst = pages + np.arange((beams - 1) * pages)
    return np.stack([src, dst], axis=1).astype(np.int64)


def custom(name: str, seed: int, dtype: str, lens, num_heads: int, num_kv_heads: int,
           head_dim: int, block_size: int, num_blocks: Optional[int] = None,
           partition_size: int = 0, manager=None) -> Workload:
    """Independent sequences with explicit context lengths (each >= 1)."""
    rng = np.random.default_rng(seed)
    return _plain(name, seed, dtype, np.asarray(lens), num_heads, num_kv_heads, head_dim,
                  block_size, rng, num_blocks=num_blocks, partition_size=partition_size,
                  manager=manager, description=f"{len(lens)} seqs, {num_heads}/{num_kv_heads} heads, D {head_dim}, "
                              f"bs {block_size}, {dtype}")


# Named workloads: the tiny case, the 8B- and 70B-shaped layers, prefix sharing,
# beams, long context, then several prompts at once.
NAMED = {
    "tiny": tiny,
    "llama3_8b": llama3_8b,
    "llama3_70b": llama3_70b,
    "prefix_share": prefix_share,
    "beam_fork": beam_fork,
    "long_context": long_context,
    "prefix_groups": prefix_groups,
}


def by_name(name: str, manager=None) -> Workload:
    return NAMED[name](manager=manager)


# ---------------------------------------------------------------------------
# values
# ---------------------------------------------------------------------------

def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def make_tensors(w: Workload, device, value_seed: Optional[int] = None) -> Dict[str, object]:
    """Draw the step's tensors on ``device`` (torch), NaN-poisoning every slot
    that holds no token before the step.  Returns a dict of torch tensors."""
    import torch
    dev = torch.device(device)
    td = torch_dtype(w.dtype)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed if value_seed is None else value_seed)

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=dev, dtype=torch.float32).to(td)

    B, Hq, Hkv, D = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim
    T = int(w.append_slots.shape[0])
    rows = B if w.query_lens is None else int(w.query_lens.sum())
    q = randn(rows, Hq, D)
    k_new = randn(T, Hkv, D)
    v_new = randn(T, Hkv, D)
    k_cache = randn(*w.k_cache_shape())
    v_cache = randn(*w.v_cache_shape())
    mask = torch.from_numpy(w.resident).to(dev)
    nan = torch.tensor(float("nan"), dtype=td, device=dev)
    nb, bs = w.num_blocks, w.block_size
    k_cache = torch.where(mask.view(nb, 1, 1, bs, 1), k_cache, nan)
    v_cache = torch.where(mask.view(nb, 1, 1, bs), v_cache, nan)
    return {
        "q": q, "k_new": k_new, "v_new": v_new,
        "k_cache": k_cache.contiguous(), "v_cache": v_cache.contiguous(),
        "block_tables": torch.from_numpy(w.block_tables).to(dev),
        "context_lens": torch.from_numpy(w.context_lens).to(dev),
        "slot_mapping": torch.from_numpy(w.append_slots).to(dev),
        "copy_pairs": torch.from_numpy(w.copy_pairs).to(dev),
        "query_start": None if w.query_lens is None else torch.from_numpy(w.query_start).to(dev),
    }
