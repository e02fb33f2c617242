"""Helpers for the GPU parity tests: device checks, host copies of device
buffers in their storage form, and the tolerance checks."""

import sys

import numpy as np
import pytest
import torch

import oracle

# Attention-output tolerances: fp32 caches max-abs 1e-5; bf16 caches max-abs
# 2e-2 and relative L2 (over all compared outputs) 5e-3.  The relative-L2
# bound is also applied to every (sequence, head) row on its own, so an error
# confined to one row can no longer hide under the norm of the whole batch.
# Measured at full size: the one bf16 rounding of the output gives a relative
# L2 of about 1.7e-3 (vector-ALU kernel, worst row 2.2e-3); the matrix-core
# kernel rounds the softmax weights to bf16 for P.V as well, 2.2e-3 (worst
# row 3.5e-3).
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
BF16_ROW_REL_L2 = 5e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_cache_350_amd as pa
    pa.lib()            # raises loudly if libpa.so is missing
    return pa


def say(*msg):
    print("[gpu-case]", *msg, flush=True)
    sys.stdout.flush()


# Parity lines printed in pytest's terminal summary (see conftest.py), so the
# worst rows of the full-size comparisons show even in a quiet run.
REPORT = []


def report(what: str, stats: dict):
    line = f"{what}: " + ", ".join(f"{k} {v:.3g}" if isinstance(v, float) else f"{k} {v}"
                                   for k, v in stats.items())
    REPORT.append(line)
    say(line)


def storage_np(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in storage form (float32, or uint16 bf16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    return t.numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality of two device tensors (NaN payloads included)."""
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    iv = {torch.bfloat16: torch.int16, torch.float32: torch.int32}[a.dtype]
    return bool(torch.equal(a.view(iv), b.view(iv)))


def row_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    """Worst (sequence, head) row of an attention output [rows, heads, D]:
    its relative L2 error and its max-abs error over max|ref|, each with the
    (row, head) where it occurs.  A row whose reference is all zeros (an
    empty context) counts its error against 1."""
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    heads = got.shape[1] if got.ndim == 3 else 1
    ref_norm = np.linalg.norm(r, axis=1)
    ref_max = np.abs(r).max(axis=1)
    rel = np.linalg.norm(g - r, axis=1) / np.where(ref_norm > 0, ref_norm, 1.0)
    mx = np.abs(g - r).max(axis=1) / np.where(ref_max > 0, ref_max, 1.0)
    i, k = int(rel.argmax()), int(mx.argmax())
    return {"worst_row_rel_l2": float(rel[i]), "worst_row_rel_l2_at": list(divmod(i, heads)),
            "worst_row_maxabs_over_maxref": float(mx[k]), "worst_row_maxabs_at": list(divmod(k, heads))}


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", f32_max_abs: float = F32_MAX_ABS):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= f32_max_abs, f"{what}: max-abs {err.max():.3g} > {f32_max_abs:.3g}"
        return {"max_abs": float(err.max())}
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert err.max() <= BF16_MAX_ABS, f"{what}: max-abs {err.max():.3g} > {BF16_MAX_ABS}"
    assert rel <= BF16_REL_L2, f"{what}: rel-L2 {rel:.3g} > {BF16_REL_L2}"
    stats = {"max_abs": float(err.max()), "rel_l2": rel}
    if got.ndim >= 2:
        rows = row_stats(got, ref)
        assert rows["worst_row_rel_l2"] <= BF16_ROW_REL_L2, \
            f"{what}: row {rows['worst_row_rel_l2_at']} rel-L2 {rows['worst_row_rel_l2']:.3g} > {BF16_ROW_REL_L2}"
        stats.update(rows)
    return stats


def sub_pool(w, t, seqs, k_cache=None, v_cache=None):
    """Host copies of only the pages the given sequences read, with their
    block-table rows renumbered into that sub-pool (input plumbing, so the
    oracle does not need the whole multi-GB pool on the host)."""
    k_cache = t["k_cache"] if k_cache is None else k_cache
    v_cache = t["v_cache"] if v_cache is None else v_cache
    bs = w.block_size
    used = []
    for b in seqs:
        n = -(-int(w.context_lens[b]) // bs)
        used.extend(int(p) for p in w.block_tables[b, :n])
    pages = sorted(set(used)) or [0]
    where = {p: i for i, p in enumerate(pages)}
    idx = torch.tensor(pages, dtype=torch.long, device=k_cache.device)
    kc = storage_np(k_cache.index_select(0, idx))
    vc = storage_np(v_cache.index_select(0, idx))
    tables = np.zeros((len(seqs), w.block_tables.shape[1]), dtype=np.int32)
    for i, b in enumerate(seqs):
        n = -(-int(w.context_lens[b]) // bs)
        tables[i, :n] = [where[int(p)] for p in w.block_tables[b, :n]]
    lens = w.context_lens[list(seqs)]
    return kc, vc, tables, lens


def oracle_decode(w, t, seqs, k_cache=None, v_cache=None):
    """Oracle decode of ``seqs`` over caches taken as they stand: only for
    caches the library has not written (as generated, or uploaded from the
    host)."""
    kc, vc, tables, lens = sub_pool(w, t, seqs, k_cache, v_cache)
    q = storage_np(t["q"])[list(seqs)]
    return oracle.decode(q, kc, vc, tables, lens, w.scale, w.block_size, w.dtype)


def run_step_updates(pa, w, t):
    """Apply the step's copy-on-write copies and appends on the GPU."""
    if len(w.copy_pairs):
        pa.copy_blocks(t["k_cache"], t["v_cache"], t["copy_pairs"])
    if len(w.append_slots):
        pa.kv_append(t["k_new"], t["v_new"], t["slot_mapping"], t["k_cache"], t["v_cache"])


def reference_after_step(w, t, seqs, scale=None):
    """The float64 oracle decode of ``seqs`` after the step's copy-on-write
    copies and appends, computed on the host before the device runs them.
    The pages those sequences read (plus the sources copied into them) are
    taken as generated; the oracle applies its own copy_blocks and kv_append
    of the same pairs and rows, renumbered into that sub-pool, so nothing
    the library writes reaches the oracle."""
    seqs = list(seqs)
    bs = w.block_size
    read = set()
    for b in seqs:
        n = -(-int(w.context_lens[b]) // bs)
        read.update(int(p) for p in w.block_tables[b, :n])
    pairs = [(int(s), int(d)) for s, d in w.copy_pairs.reshape(-1, 2) if int(d) in read]
    pages = sorted(read | {s for s, _ in pairs}) or [0]
    where = {p: i for i, p in enumerate(pages)}
    idx = torch.tensor(pages, dtype=torch.long, device=t["k_cache"].device)
    kc = storage_np(t["k_cache"].index_select(0, idx))
    vc = storage_np(t["v_cache"].index_select(0, idx))
    kc, vc = oracle.copy_blocks(kc, vc, np.array([[where[s], where[d]] for s, d in pairs], np.int64).reshape(-1, 2))
    slots = np.asarray(w.append_slots, dtype=np.int64)
    keep = np.array([s >= 0 and int(s) // bs in read for s in slots], dtype=bool)
    sub = np.array([where[int(s) // bs] * bs + int(s) % bs for s in slots[keep]], dtype=np.int64)
    kc, vc = oracle.kv_append(storage_np(t["k_new"])[keep], storage_np(t["v_new"])[keep], sub, kc, vc, bs)
    tables = np.zeros((len(seqs), w.block_tables.shape[1]), dtype=np.int32)
    for i, b in enumerate(seqs):
        n = -(-int(w.context_lens[b]) // bs)
        tables[i, :n] = [where[int(p)] for p in w.block_tables[b, :n]]
    q = storage_np(t["q"])[seqs]
    return oracle.decode(q, kc, vc, tables, w.context_lens[seqs], w.scale if scale is None else scale, bs, w.dtype)


def step_and_reference(pa, w, t, seqs, scale=None):
    """reference_after_step (with the workload's scale, or ``scale``), then
    the step's copies and appends on the GPU."""
    ref = reference_after_step(w, t, seqs, scale)
    run_step_updates(pa, w, t)
    return ref
