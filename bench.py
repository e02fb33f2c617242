"""Benchmark: one paged-decode step per iteration on one MI355X.

A step is the whole data-parallel path over one synthetic batch: the KV
append of every sequence's newest token and paged decode attention over all
cached tokens.  By default the append runs inside the decode kernel
(pa_decode_append: partition kernel + merge kernel on the split path);
--step separate times pa_kv_append followed by pa_decode instead.  Inputs are
resident in HBM before timing starts.

Default workload: the Llama-3-8B-shaped layer -- 64 sequences, 32 query / 8
kv heads, head_dim 128, block 16, bf16, context lengths uniform in
[512, 4096], pool = pages needed + 10 %, page ids randomly permuted.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line.  `value` is KV bytes read per step (every context
token's K and V row once per kv head; for workloads whose sequences share
pages, every distinct page slot once -- the bytes a step must bring from HBM)
divided by the wall time per step.  `roofline` times the dominant kernel
alone: 200 back-to-back launches between one pair of HIP events on the
stream the library launches on.  `step_timing` gives the median, p10 and p90
of single steps, warm (back to back) and cold (L2 and the Infinity Cache
evicted before each step).  `cpu_baseline` times the float64 oracle on the
host cores (one worker process per core), on a bounded sample of the same
batch.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, published peak
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak, published
METRIC = "paged-decode KV GB/s read (% of MI355X HBM peak) and decode seqs/sec"


def _args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--step", default="fused", choices=["fused", "separate", "prefix"],
                    help="fused: the append runs inside the decode kernel (pa_decode_append); "
                         "separate: pa_kv_append, then pa_decode; prefix: pa_decode_shared_prefix "
                         "(append fused) with the longest prefix the block tables share "
                         "(whole pages; the library's default partition unless --partition-size is given)")
    ap.add_argument("--reuse", default="auto", choices=["auto", "stream", "shared"],
                    help="K/V load path (auto: shared when the workload's sequences share pages)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="override the library default (0 default, -1 single pass)")
    ap.add_argument("--samples", type=int, default=200,
                    help="single steps timed warm and cold, and back-to-back launches of the dominant kernel "
                         "(at least --steps); fewer keep a profiled run short")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time for the oracle baseline sample")
    ap.add_argument("--mode", default="decode", choices=["decode", "copy_probe", "copy_calib",
                                                         "blockmgr", "capacity", "prefix", "multi",
                                                         "append_bulk", "read_calib"],
                    help="copy_probe: time pa_copy_blocks on an eager fork of a 32,768-token "
                         "prompt to 7 beams (7,168 pages of 32 tokens, K and V); copy_calib: "
                         "the same number of page copies with 7,168 distinct sources (a plain "
                         "copy of known size, used to scale rocprofv3 traffic counters); "
                         "blockmgr: host time of one decode step's page bookkeeping (append "
                         "for every sequence + block tables), native manager vs the Python one "
                         "(no GPU needed); capacity: KV waste and concurrent capacity, paged vs "
                         "contiguous pre-allocation, measured with the native allocator (no GPU); "
                         "prefix: prefix caching on a multi-tenant request stream, native manager "
                         "vs the oracle (no GPU); multi: multi-query attention on the "
                         "speculative-verification batch (5 queries per sequence); append_bulk: "
                         "pa_kv_append at prefill sizes; read_calib: streaming reads of a known "
                         "size with and without the non-temporal bit (to scale traffic counters)")
    ap.add_argument("--multi-workload", default="spec_verify", choices=["spec_verify", "prompt_chunk"],
                    help="multi mode: speculative verification (5 queries per sequence, HBM-bound) or a "
                         "prompt chunk (512 queries per sequence over 3,584 cached tokens, matrix-bound)")
    ap.add_argument("--requests", type=int, default=2000, help="prefix mode: requests in the stream")
    ap.add_argument("--oracle-requests", type=int, default=400,
                    help="prefix mode: leading requests the oracle replays (CPU baseline sample)")
    return ap.parse_args(argv)


def _src_digest():
    """Digest of every HIP source and header of the library (a counter summary
    taken on other sources no longer describes the kernels that run)."""
    csrc = os.path.join(ROOT, "paged_kv_cache_350_amd", "csrc")
    h = hashlib.sha256()
    for n in sorted(os.listdir(csrc)):
        if n.endswith((".hip", ".h")):
            with open(os.path.join(csrc, n), "rb") as f:
                h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_name, workload, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_name}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def _host(t):
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ---- CPU baseline: the float64 oracle, process-parallel over the host cores
#
# Workers are spawned interpreters (fresh processes that never touch the
# GPU); the cache pages the batch reads are handed over once in shared host
# memory, and every task is one whole sequence.

_CPU = {}


def _cpu_worker_init(shm_name, kshape, vshape, kdtype, q, tables, lens, scale, bs, dtype):
    from multiprocessing import shared_memory
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:           # pragma: no cover - threadpoolctl missing
        pass
    shm = shared_memory.SharedMemory(name=shm_name)    # the parent owns (and unlinks) it
    nk = int(np.prod(kshape)) * np.dtype(kdtype).itemsize
    _CPU.update(shm=shm, q=q, tables=tables, lens=lens, scale=scale, bs=bs, dtype=dtype,
                kc=np.ndarray(kshape, dtype=kdtype, buffer=shm.buf[:nk]),
                vc=np.ndarray(vshape, dtype=kdtype, buffer=shm.buf[nk:]))


def _cpu_worker_run(b):
    import oracle
    c = _CPU
    oracle.decode(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], c["scale"], c["bs"], c["dtype"], seqs=[b])
    return b


def cpu_baseline(w, t, target_s):
    """Oracle (float64, host) over whole sequences of the batch, one process
    per host core (one BLAS thread each), about `target_s` seconds of wall
    time: the batch's sequences are queued round after round."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    import torch
    bs = w.block_size
    seqs = [b for b in range(w.num_seqs) if int(w.context_lens[b]) > 0]
    pages = sorted({int(p) for b in seqs for p in w.block_tables[b, :-(-int(w.context_lens[b]) // bs)]})
    where = np.zeros(w.num_blocks, dtype=np.int64)
    where[pages] = np.arange(len(pages))
    idx = torch.tensor(pages, dtype=torch.long, device=t["k_cache"].device)
    kc = _host(t["k_cache"].index_select(0, idx))
    vc = _host(t["v_cache"].index_select(0, idx))
    tables = np.zeros_like(w.block_tables)
    for b in seqs:
        n = -(-int(w.context_lens[b]) // bs)
        tables[b, :n] = where[w.block_tables[b, :n]]
    q = _host(t["q"])
    batch_bytes = int(sum(int(w.context_lens[b]) for b in seqs)) * w.kv_bytes_per_token()
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    if any("rocprof" in v.lower() for k, v in os.environ.items() if k in ("LD_PRELOAD", "HSA_TOOLS_LIB")):
        # under a profiler every new process would load its tool library
        # (and open the GPU): no worker processes then
        return None
    shm = shared_memory.SharedMemory(create=True, size=kc.nbytes + vc.nbytes)
    try:
        np.ndarray(kc.shape, dtype=kc.dtype, buffer=shm.buf[:kc.nbytes])[...] = kc
        np.ndarray(vc.shape, dtype=vc.dtype, buffer=shm.buf[kc.nbytes:])[...] = vc
        kshape, vshape, kdtype = kc.shape, vc.shape, kc.dtype
        del kc, vc
        ctx = mp.get_context("spawn")
        with ctx.Pool(cores, initializer=_cpu_worker_init,
                      initargs=(shm.name, kshape, vshape, kdtype, q, tables, w.context_lens, w.scale, bs,
                                w.dtype)) as pool:
            # a worker that cannot start would leave map() waiting forever:
            # every round has a deadline
            pool.map_async(_cpu_worker_run, seqs, chunksize=1).get(timeout=120)   # warm-up (imports, page-in)
            t0 = time.perf_counter()
            pool.map_async(_cpu_worker_run, seqs, chunksize=1).get(timeout=120)
            first = time.perf_counter() - t0
            rounds = max(1, int(round(target_s / max(first, 1e-3))))
            t0 = time.perf_counter()
            pool.map_async(_cpu_worker_run, seqs * rounds, chunksize=1).get(timeout=10 * target_s + 120)
            wall = time.perf_counter() - t0
    finally:
        shm.close()
        shm.unlink()
    done = rounds * len(seqs)
    return {
        "value": round(rounds * batch_bytes / wall / 1e9, 4), "unit": "GB/s",
        "seqs_per_s": round(done / wall, 3), "cores": cores, "kind": "oracle",
        "sample": f"{rounds} round(s) of the whole {w.name} batch ({done} sequences, "
                  f"{rounds * batch_bytes / 1e6:.1f} MB of KV), float64 numpy oracle, {cores} worker "
                  f"processes with one BLAS thread each, {wall:.1f} s wall",
        "host_cores_available": len(os.sched_getaffinity(0)),
    }


def stream_read_gbps(torch, pa, nbytes, reps=20):
    """Achievable-read reference: libpa's streaming-read probe (non-temporal
    16-byte loads, 2048 workgroups) over a buffer of ``nbytes``."""
    nbytes = nbytes // 16 * 16
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pa.probe_stream_read(x, sink)
    stream = torch.cuda.current_stream()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        pa.probe_stream_read(x, sink)
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del x
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def copy_probe(a, torch, pa, W) -> int:
    """Eager-fork page copy: 7 x 1024 pages (bs 32, 8 kv heads, D 128, bf16).
    In copy_calib mode every source page is distinct, so every byte read
    comes from HBM once."""
    pairs = W.copy_probe()
    if a.mode == "copy_calib":
        n = len(pairs)
        pairs = np.stack([np.arange(n), n + np.arange(n)], axis=1).astype(np.int64)
    nb = int(pairs.max()) + 1
    kc = torch.zeros(nb, 8, 16, 32, 8, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(nb, 8, 128, 32, dtype=torch.bfloat16, device="cuda")
    mp = torch.from_numpy(pairs).cuda()
    for _ in range(a.warmup):
        pa.copy_blocks(kc, vc, mp)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(a.steps):
        pa.copy_blocks(kc, vc, mp)
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1e3 / a.steps
    page_bytes = 2 * 8 * 128 * 32 * 2          # K + V of one page
    moved = len(pairs) * page_bytes * 2        # read + write
    print(json.dumps({"mode": a.mode, "pairs": int(len(pairs)), "bytes_read": moved // 2,
                      "bytes_written": moved // 2, "avg_us": round(us, 2),
                      "gbps_read_plus_write": round(moved / (us * 1e-6) / 1e9, 1),
                      "steps": a.steps}), flush=True)
    return 0


def append_bulk(a, torch, pa, W) -> int:
    """pa_kv_append at prefill sizes: the 32,768-token prompt of the beam
    workload written into 1,024 pages of 32 tokens (page order permuted), and
    the prefix workload's suffix prefill (every suffix token but each
    sequence's newest).  Bytes moved = rows read + the same bytes written."""
    res = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(5)

    def time_append(name, k, v, slots, kc, vc):
        fn = lambda: pa.kv_append(k, v, slots, kc, vc)        # noqa: E731
        for _ in range(max(a.warmup, 1)):
            fn()
        ms = _loop_ms(torch, torch.cuda.current_stream(), fn, max(a.steps, 20))
        moved = 2 * (k.numel() + v.numel()) * k.element_size()
        res[name] = {"tokens": int(k.shape[0]), "bytes_read_plus_written": moved, "avg_us": round(ms * 1e3, 2),
                     "gbps_read_plus_write": round(moved / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    # beam prompt: 32,768 tokens, block 32, 8 kv heads, D 128, bf16
    T, bs, hkv, d = 32768, 32, 8, 128
    pages = T // bs
    nb = pages + pages // 10
    order = torch.from_numpy(np.random.default_rng(5).permutation(nb)[:pages].astype(np.int64)).cuda()
    slots = (order.repeat_interleave(bs) * bs + torch.arange(bs, device="cuda").repeat(pages)).contiguous()
    k = torch.randn(T, hkv, d, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(T, hkv, d, generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.zeros(nb, hkv, d // 8, bs, 8, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(nb, hkv, d, bs, dtype=torch.bfloat16, device="cuda")
    time_append("beam_prompt_32768", k, v, slots, kc, vc)
    del k, v, kc, vc

    # prefix workload: the suffix prefill after the copy-on-write fork
    w = W.prefix_share()
    t = W.make_tensors(w, "cuda")
    newest = {}
    for i, b in enumerate(w.append_seq.tolist()):
        newest[b] = i
    older = torch.tensor([i for i in range(len(w.append_seq)) if i not in set(newest.values())],
                         dtype=torch.long, device="cuda")
    time_append("prefix_suffix_prefill", t["k_new"].index_select(0, older).contiguous(),
                t["v_new"].index_select(0, older).contiguous(),
                t["slot_mapping"].index_select(0, older).contiguous(), t["k_cache"], t["v_cache"])
    print(json.dumps({"mode": "append_bulk", "digest": _src_digest(), "steps": max(a.steps, 20),
                      "results": res}), flush=True)
    return 0


def read_calib(a, torch, pa) -> int:
    """Streaming reads of a known size (1 GiB per dispatch), with and without
    the non-temporal bit: what FETCH_SIZE reads for them scales the counter
    for kernels whose loads are streaming (the decode kernels) or ordinary."""
    nbytes = 1 << 30
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for nt in (True, False):
        for _ in range(max(a.steps, 1)):
            pa.probe_stream_read(x, sink, nontemporal=nt)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "read_calib", "bytes_per_dispatch": nbytes, "dispatches_each": max(a.steps, 1)}),
          flush=True)
    return 0


def blockmgr_bench(a) -> int:
    """Decode-step bookkeeping of the Llama-3-70B-shaped batch: every one of
    the 256 sequences appends a token, then the int32 block tables and
    context lengths the kernels take are built.  Native manager (libpa) vs
    the host Python manager, same pool and page order."""
    import paged_kv_cache_350_amd as pa
    import workloads as W
    w = W.llama3_70b()
    steps = a.steps
    seqs = list(range(w.num_seqs))
    lens = (w.context_lens.astype(np.int64) - 1).tolist()
    grow = w.num_seqs * (steps // w.block_size + 2)
    nb = w.num_blocks + grow
    order = np.random.default_rng(w.seed).permutation(nb)
    maxb = -(-(int(max(lens)) + steps) // w.block_size)

    def run(mgr, native):
        for b, L in zip(seqs, lens):
            mgr.allocate(b, L)
        page_lists = mgr.tables if hasattr(mgr, "lengths") else getattr(mgr, "pages", None)
        lengths = mgr.lengths if hasattr(mgr, "lengths") else getattr(mgr, "length", None)
        if native:
            ids = np.asarray(seqs, dtype=np.int64)
            tables, ctx = mgr.block_tables(ids, maxb, pad_page=0)
        t0 = time.perf_counter()
        for _ in range(steps):
            if native:        # the tables are kept current in place
                slots, copies = mgr.append(ids, tables, ctx)
            else:
                slots = np.array([mgr.append_token(b) for b in seqs], dtype=np.int64)
                tables = np.zeros((len(seqs), maxb), dtype=np.int32)
                for i, b in enumerate(seqs):
                    pg = page_lists[b]
                    tables[i, :len(pg)] = pg
                ctx = np.array([lengths[b] for b in seqs], dtype=np.int32)
        return (time.perf_counter() - t0) / steps * 1e6, tables, ctx, slots

    from oracle.prefix_cache import PrefixCachingPool
    nat_us, t_n, c_n, s_n = run(pa.NativeBlockManager(nb, w.block_size, free_order=order), True)
    py_us, t_p, c_p, s_p = run(W.BlockManager(nb, w.block_size, free_order=order), False)
    or_us, t_o, c_o, s_o = run(PrefixCachingPool(nb, w.block_size, free_order=order.tolist()), False)
    same = bool(np.array_equal(t_n, t_p) and np.array_equal(c_n, c_p) and np.array_equal(s_n, s_p) and
                np.array_equal(t_n, t_o) and np.array_equal(c_n, c_o) and np.array_equal(s_n, s_o))
    print(json.dumps({"mode": "blockmgr", "workload": w.name, "num_seqs": w.num_seqs, "steps": steps,
                      "native_us_per_step": round(nat_us, 2), "host_python_us_per_step": round(py_us, 2),
                      "speedup": round(py_us / nat_us, 1), "identical_tables_slots": same,
                      "pool_pages": nb, "max_blocks_per_seq": maxb,
                      "cpu_baseline": {"value": round(or_us, 2), "unit": "us/step", "cores": 1, "kind": "oracle",
                                       "sample": f"{steps} steps of the same bookkeeping by the oracle's "
                                                 f"plain page pool (oracle/prefix_cache.py)"}}), flush=True)
    return 0 if same else 1


def capacity_bench(a) -> int:
    """KV waste of every named workload and concurrent capacity of a whole
    Llama-3-shaped model's KV on one MI355X, paged (native allocator) vs a
    contiguous runtime that reserves each request's maximum length."""
    from paged_kv_cache_350_amd import capacity as C
    import workloads as W
    reserve = {"tiny": 64, "llama3_8b": 4096, "llama3_70b": 8192, "prefix_share": 10512,
               "beam_fork": 32774, "long_context": 32768}
    usage = {}
    for name in reserve:
        w = W.by_name(name)
        if name == "prefix_share":
            u = C.measure_usage(w.context_lens, w.block_size, reserve[name], prompt=10000)
            flat = C.measure_usage(w.context_lens, w.block_size, reserve[name])
        elif name == "beam_fork":
            u = C.measure_usage(w.context_lens, w.block_size, reserve[name], prompt=32768 + 5)
            flat = C.measure_usage(w.context_lens, w.block_size, reserve[name])
        else:
            u = flat = C.measure_usage(w.context_lens, w.block_size, reserve[name])
        d = u.as_dict()
        d["reserve_tokens"] = reserve[name]
        if u is not flat:
            d["sharing_saving_vs_unshared_paged"] = round(1 - u.paged_tokens / flat.paged_tokens, 4)
            d["sharing_saving_vs_contiguous"] = round(1 - u.paged_tokens / u.contiguous_tokens, 4)
        usage[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}
    kv_budget = 250e9           # bytes of HBM given to the KV cache on a 288 GB MI355X
    models = {"llama3_8b": (32, 4096), "llama3_70b": (80, 8192)}
    cap = {}
    for name, (layers, res) in models.items():
        per_tok = C.kv_bytes_per_token(layers, 8, 128, 2)
        tokens = int(kv_budget // per_tok)
        paged = C.paged_capacity(tokens, 16, C.sample_lengths(name, 4096, seed=5))
        contig = C.contiguous_capacity(tokens, res)
        cap[name] = {"layers": layers, "kv_bytes_per_token": per_tok, "budget_tokens": tokens,
                     "reserve_tokens": res, "paged_sequences": paged, "contiguous_sequences": contig,
                     "ratio": round(paged / contig, 2)}
    print(json.dumps({"mode": "capacity", "kv_budget_bytes": kv_budget, "usage": usage,
                      "capacity": cap}), flush=True)
    return 0


def prefix_bench(a) -> int:
    """Prefix caching on a multi-tenant request stream: share of prompt
    tokens whose K/V was already cached, pages held with and without
    caching, and the native manager's host cost per admission next to the
    oracle's on a bounded sample (with identical decisions)."""
    import paged_kv_cache_350_amd as pa
    from paged_kv_cache_350_amd import capacity as C
    import workloads.requests as R
    from oracle.prefix_cache import PrefixCachingPool
    bs, live_max = 16, 100
    reqs = R.tenant_requests(num_tenants=8, num_requests=a.requests, seed=7)
    arrays = [np.asarray(t, dtype=np.int32) for _, t in reqs]   # token ids as a serving loop holds them
    per_tok = C.kv_bytes_per_token(32, 8, 128, 2)              # Llama-3-8B-shaped KV
    nb = int(250e9 // per_tok) // bs                           # 250 GB of HBM for KV

    def run(mgr, prompt_api, limit, native=True):
        """Admissions are timed without reading the pages back (a serving
        loop reads them through the block tables); the oracle's decisions
        and the native manager's are compared on the leading sample."""
        live, cached_sum, prompt_sum, peak, t_adm, t_free = [], 0, 0, 0, 0.0, 0.0
        decisions = []
        for i, (_, toks) in enumerate(reqs[:limit]):
            if len(live) == live_max:                          # the oldest request finishes
                t0 = time.perf_counter()
                mgr.free_sequence(live.pop(0))
                t_free += time.perf_counter() - t0
            t0 = time.perf_counter()
            if not native:
                cached = mgr.allocate_prompt(i, toks)[1]
            elif prompt_api:
                cached = mgr.allocate_prompt(i, arrays[i], return_pages=False)
            else:
                mgr.allocate(i, len(toks), return_pages=False)
                cached = 0
            t_adm += time.perf_counter() - t0
            if i < sample:
                decisions.append((list(mgr.pages[i] if not native else mgr.pages(i)), cached))
            live.append(i)
            cached_sum += cached
            prompt_sum += len(toks)
            held = nb - (mgr.num_free() if callable(getattr(mgr, "num_free", None)) else len(mgr.free))
            peak = max(peak, held)
        n = max(limit, 1)
        return {"cached_tokens": cached_sum, "prompt_tokens": prompt_sum, "peak_pages": peak,
                "us_per_admission": t_adm / n * 1e6, "us_per_free": t_free / n * 1e6}, decisions

    sample = min(a.oracle_requests, len(reqs))
    nat, nat_dec = run(pa.NativeBlockManager(nb, bs), True, len(reqs))
    flat, _ = run(pa.NativeBlockManager(nb, bs), False, len(reqs))
    t0 = time.perf_counter()
    orc, orc_dec = run(PrefixCachingPool(nb, bs), True, sample, native=False)
    oracle_s = time.perf_counter() - t0
    same = orc_dec == nat_dec[:sample]
    print(json.dumps({
        "mode": "prefix", "requests": len(reqs), "tenants": 8, "block_size": bs, "live_max": live_max,
        "pool_pages": nb, "cached_token_fraction": round(nat["cached_tokens"] / nat["prompt_tokens"], 4),
        "peak_pages_cached": nat["peak_pages"], "peak_pages_uncached": flat["peak_pages"],
        "memory_saving": round(1 - nat["peak_pages"] / flat["peak_pages"], 4),
        "prefill_kv_bytes_skipped": nat["cached_tokens"] * per_tok,
        "native_us_per_admission": round(nat["us_per_admission"], 2),
        "native_us_per_free": round(nat["us_per_free"], 2),
        "uncached_native_us_per_admission": round(flat["us_per_admission"], 2),
        "identical_decisions_on_sample": same,
        "cpu_baseline": {"value": round(orc["us_per_admission"], 2), "unit": "us/admission", "cores": 1,
                         "kind": "oracle", "sample": f"first {sample} requests of the stream",
                         "seconds": round(oracle_s, 2)}}), flush=True)
    return 0 if same else 1


def multi_bench(a, torch, pa, W) -> int:
    """Multi-query step on the speculative-verification batch: every
    sequence's new tokens appended and attended to -- in one launch
    (pa_decode_multi_append, --step fused, the default) or as pa_kv_append
    then pa_decode_multi (--step separate).  The roofline figure uses the
    whole pa_decode_multi call as the launch (one kernel in one pass; with a
    split the merge kernel too, which the rocprofv3 summary separates)."""
    import oracle
    chunk = a.multi_workload == "prompt_chunk"
    w = W.prompt_chunk() if chunk else W.spec_verify()
    t = W.make_tensors(w, "cuda")
    reuse = a.reuse if a.reuse != "auto" else "stream"
    ps_req = 0 if a.partition_size is None else a.partition_size
    P = pa.decode_multi_partition_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.max_context_len,
                                       w.max_query_len, ps_req)
    T = int(w.query_lens.sum())
    nws = pa.decode_multi_workspace_size(w.num_seqs, T, w.num_heads, w.num_kv_heads, w.head_dim,
                                         w.max_context_len, w.max_query_len, P)
    ws = torch.empty(max(nws // 4, 1), dtype=torch.float32, device="cuda")
    out = torch.empty_like(t["q"])
    stream = torch.cuda.current_stream()

    fused = a.step == "fused"
    app = dict(k_new=t["k_new"], v_new=t["v_new"]) if fused else {}

    def step():
        if not fused:
            pa.kv_append(t["k_new"], t["v_new"], t["slot_mapping"], t["k_cache"], t["v_cache"])
        pa.decode_multi(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                        t["query_start"], w.scale, w.max_context_len, w.max_query_len, out=out,
                        partition_size=P if P > 0 else -1, workspace=ws, reuse=reuse, **app)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: warmup done, timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # each launch alone, back to back, one event pair around the loop
    nloop = max(a.steps, a.samples)
    append_ms = _loop_ms(torch, stream, lambda: pa.kv_append(t["k_new"], t["v_new"], t["slot_mapping"],
                                                            t["k_cache"], t["v_cache"]), nloop)
    multi_ms = _loop_ms(torch, stream, lambda: pa.decode_multi(
        t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"], t["query_start"], w.scale,
        w.max_context_len, w.max_query_len, out=out, partition_size=P if P > 0 else -1, workspace=ws,
        reuse=reuse, **app), nloop)
    kv_bytes = w.algorithmic_kv_bytes()       # every context token once per kv head (one column group)
    flops = w.multi_flops()
    ms_per_step = wall * 1e3 / a.steps
    achieved = kv_bytes / (multi_ms * 1e-3) / 1e9
    digest = _src_digest()

    # CPU baseline: the oracle on whole sequences, about cpu_seconds of work
    cpu = None
    if not a.no_cpu_baseline:
        kc0, vc0, q = _host(t["k_cache"]), _host(t["v_cache"]), _host(t["q"])
        done = nbytes = 0
        elapsed = 0.0
        for b in range(w.num_seqs):
            t1 = time.perf_counter()
            oracle.decode_multi(q, kc0, vc0, w.block_tables, w.context_lens, w.query_start, w.scale,
                                w.block_size, w.dtype, seqs=[b])
            elapsed += time.perf_counter() - t1
            done += 1
            nbytes += int(w.context_lens[b]) * w.kv_bytes_per_token()
            if elapsed >= a.cpu_seconds:
                break
        if chunk:       # the sequences are alike: flops in proportion
            cpu = {"value": round(flops * done / w.num_seqs / elapsed / 1e9, 3), "unit": "GFLOP/s", "cores": 1,
                   "kind": "oracle", "sample": f"{done} whole sequences of the {w.name} batch, float64 numpy "
                                               f"oracle, {elapsed:.1f} s of CPU time"}
        else:
            cpu = {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                   "sample": f"{done} whole sequences of the {w.name} batch, float64 numpy oracle, "
                             f"{elapsed:.1f} s of CPU time"}
    kname = "decode_multi" + ("_single" if P <= 0 else " partition + merge")
    if chunk:
        # matrix-bound: 512 queries per sequence make the product dense
        tflops = flops / (multi_ms * 1e-3) / 1e12
        rec = {
            "metric": "multi-query paged attention TFLOP/s (chunked prefill)",
            "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "prompt_tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
            "config": {"workload": w.name, "description": w.description, "num_seqs": w.num_seqs,
                       "query_tokens": T, "max_query_len": w.max_query_len,
                       "sum_context_tokens": int(w.context_lens.sum()), "max_context_len": w.max_context_len,
                       "partition_size": P, "flops_per_step": flops, "kv_bytes_per_step": kv_bytes,
                       "step": a.step},
            "kernels_avg_us": {"kv_append": None if fused else round(append_ms * 1e3, 2),
                               kname: round(multi_ms * 1e3, 2)},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "kernel": kname, "avg_launch_us": round(multi_ms * 1e3, 2),
                         "algorithmic_flops_per_launch": flops, "source_digest": digest},
            "cpu_baseline": cpu,
        }
        print(json.dumps(rec), flush=True)
        return 0
    rec = {
        "metric": "multi-query paged attention KV GB/s read (speculative verification)",
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "verified_tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "config": {"workload": w.name, "description": w.description, "num_seqs": w.num_seqs,
                   "query_tokens": T, "max_query_len": w.max_query_len,
                   "sum_context_tokens": int(w.context_lens.sum()), "max_context_len": w.max_context_len,
                   "partition_size": P, "reuse": reuse, "kv_bytes_per_step": kv_bytes, "step": a.step},
        "kernels_avg_us": {"kv_append": None if fused else round(append_ms * 1e3, 2),
                           kname: round(multi_ms * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": _traffic("decode_multi", w.name, digest) if P <= 0 else None,
                     "kernel": kname, "avg_launch_us": round(multi_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": kv_bytes, "source_digest": digest},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def main(argv=None) -> int:
    a = _args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the library has no multi-GPU "
                                   "path (how it would shard is described in the design notes)",
                          "n_gpus": a.gpus}), flush=True)
        return 2

    if a.mode == "blockmgr":
        return blockmgr_bench(a)
    if a.mode == "capacity":
        return capacity_bench(a)
    if a.mode == "prefix":
        return prefix_bench(a)

    import torch
    import paged_kv_cache_350_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 1
    pa.lib()
    torch.cuda.set_device(0)
    if a.mode in ("copy_probe", "copy_calib"):
        return copy_probe(a, torch, pa, W)
    if a.mode == "multi":
        return multi_bench(a, torch, pa, W)
    if a.mode == "append_bulk":
        return append_bulk(a, torch, pa, W)
    if a.mode == "read_calib":
        return read_calib(a, torch, pa)
    w = W.by_name(a.workload)
    ps_req = w.partition_size if a.partition_size is None else a.partition_size
    t = W.make_tensors(w, "cuda")
    if len(w.copy_pairs):
        pa.copy_blocks(t["k_cache"], t["v_cache"], t["copy_pairs"])
    # Set-up: every token the workload appends except each sequence's newest
    # (for the prefix workload that is the rest of each suffix, its prefill).
    # The timed decode step appends the newest token of each sequence --
    # rows [B, Hkv, D] plus its slot, -1 for a sequence that appends nothing --
    # and decodes; rewriting a slot with the same row is idempotent.
    newest = {}
    for i, b in enumerate(w.append_seq.tolist()):
        newest[b] = i
    older = [i for i in range(len(w.append_seq)) if i not in set(newest.values())]
    if older:
        oi = torch.tensor(older, dtype=torch.long, device="cuda")
        pa.kv_append(t["k_new"].index_select(0, oi).contiguous(),
                     t["v_new"].index_select(0, oi).contiguous(),
                     t["slot_mapping"].index_select(0, oi).contiguous(), t["k_cache"], t["v_cache"])
    step_k = torch.zeros(w.num_seqs, w.num_kv_heads, w.head_dim, dtype=t["k_new"].dtype, device="cuda")
    step_v = torch.zeros_like(step_k)
    slots = np.full(w.num_seqs, -1, dtype=np.int64)
    for b, i in newest.items():
        step_k[b] = t["k_new"][i]
        step_v[b] = t["v_new"][i]
        slots[b] = w.append_slots[i]
    step_slots = torch.from_numpy(slots).cuda()
    fused = a.step in ("fused", "prefix")
    torch.cuda.synchronize()

    # the load path a caller picks: its block manager knows whether pages are shared
    reuse = a.reuse if a.reuse != "auto" else ("shared" if w.extra.get("shared_pages") else "stream")
    prefix = a.step == "prefix"
    if prefix:
        reuse = "shared"
        P = ps_req if ps_req else 0      # 0: the library's default for this call
        # host bookkeeping, as a block manager would know it: the leading
        # block-table entries every sequence shares, in whole pages
        shared_len = pa.shared_prefix_len(w.block_tables, w.context_lens, w.block_size)
        groups = w.extra.get("groups")
        if groups:
            # several prompts: each group's own shared length, per group and per sequence
            gsl = [pa.shared_prefix_len(w.block_tables[g0:g0 + gn], w.context_lens[g0:g0 + gn], w.block_size)
                   for g0, gn in groups]
            seq_sl = np.zeros(w.num_seqs, dtype=np.int32)
            for (g0, gn), S in zip(groups, gsl):
                seq_sl[g0:g0 + gn] = S
            garr = dict(group_start=torch.tensor([g0 for g0, _ in groups] + [sum(groups[-1])], dtype=torch.int32,
                                                 device="cuda"),
                        group_shared_len=torch.tensor(gsl, dtype=torch.int32, device="cuda"),
                        seq_shared_len=torch.from_numpy(seq_sl).cuda(),
                        max_group_size=max(gn for _, gn in groups), max_shared_len=max(gsl))
            shared_len = gsl
    else:
        P = pa.decode_partition_size(w.num_seqs, w.num_kv_heads, w.max_context_len, ps_req, reuse)
        shared_len = None
        groups = None
    split = P > 0
    out = torch.empty_like(t["q"])
    if prefix and groups:
        nws = pa.lib().pa_decode_shared_prefix_groups_workspace_size(w.num_seqs, w.num_heads, w.head_dim,
                                                                     w.max_context_len, P)
        ws = torch.empty(nws // 4, dtype=torch.float32, device="cuda")
    elif prefix:
        nws = pa.shared_prefix_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                              w.max_context_len, shared_len, P)
        ws = torch.empty(nws // 4, dtype=torch.float32, device="cuda")
    else:
        ws = pa.make_workspace(t["q"], w.num_kv_heads, w.max_context_len, P, reuse) if split else None
    kernel_name = "decode_mfma" if (a.kernel == "mfma" or (a.kernel == "auto" and w.dtype == "bf16")) \
        else "decode_valu"
    main_name = ("decode_shared_prefix_groups" if groups else "decode_shared_prefix") if prefix else kernel_name + ("_partition" if split else "_single")
    stream = torch.cuda.current_stream()
    app = dict(k_new=step_k, v_new=step_v, slot_mapping=step_slots) if fused else {}

    def run_partition():
        pa.decode_partition(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                            w.scale, w.max_context_len, P, ws, kernel=a.kernel, reuse=reuse, **app)

    def run_reduce():
        pa.decode_reduce(ws, t["context_lens"], out, w.max_context_len, P)

    def run_append():
        pa.kv_append(step_k, step_v, step_slots, t["k_cache"], t["v_cache"])

    def run_decode():
        if prefix and groups:
            pa.decode_shared_prefix_groups(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                           t["context_lens"], w.scale, w.max_context_len, partition_size=P,
                                           out=out, workspace=ws, **garr, **app)
        elif prefix:
            pa.decode_shared_prefix(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                    w.scale, w.max_context_len, shared_len, P, out=out, workspace=ws, **app)
        elif split:
            run_partition()
            run_reduce()
        elif fused:
            pa.decode_append(step_k, step_v, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                             t["context_lens"], w.scale, w.max_context_len, slot_mapping=step_slots,
                             out=out, partition_size=-1, kernel=a.kernel, reuse=reuse)
        else:
            pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                      w.scale, w.max_context_len, out=out, partition_size=-1, kernel=a.kernel, reuse=reuse)

    def step():
        if not fused:
            run_append()
        run_decode()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: warmup done, timing {a.steps} steps", file=sys.stderr, flush=True)

    # timed region: exactly `steps` steps, synchronised on both sides; one
    # event pair on the library's stream around the same back-to-back steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_event_ms = e0.elapsed_time(e1) / a.steps

    # The dominant kernel alone, back to back, one event pair around the loop:
    # the partition kernel of a split step; otherwise the decode call (one
    # kernel, or for a single pass of 12-wave workgroups over many pairs with
    # the append, the append launch plus the decode kernel; the shared-prefix
    # call is its three launches).
    nloop = max(a.steps, a.samples)
    main_ms = _loop_ms(torch, stream, run_partition if (split and not prefix) else run_decode, nloop)
    reduce_ms = _loop_ms(torch, stream, run_reduce, nloop) if split and not prefix else None
    append_ms = _loop_ms(torch, stream, run_append, nloop) if not fused else None

    # per-step distributions, warm (back to back) and cold (caches evicted
    # by a write and a read of 1 GiB each before every step, outside the events)
    nsamp = max(a.samples, 1)
    warm = _step_samples(torch, stream, step, nsamp)
    evict = _Evictor(torch, pa, 1 << 30)
    cold = _step_samples(torch, stream, step, nsamp, before=evict)
    del evict

    shared = bool(w.extra.get("shared_pages"))
    logical = w.algorithmic_kv_bytes()
    unique = w.unique_kv_bytes() if shared else logical
    kv_bytes = unique          # bytes a step must bring from HBM at least once
    ms_per_step = wall * 1e3 / a.steps
    gbps = kv_bytes / (ms_per_step * 1e-3) / 1e9

    digest = _src_digest()
    achieved = kv_bytes / (main_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": _traffic(main_name, w.name, digest),
        "kernel": main_name,
        "avg_launch_us": round(main_ms * 1e3, 2),
        "algorithmic_bytes_per_launch": kv_bytes,
        "bytes_basis": "unique" if shared else "every context token once per kv head",
        "source_digest": digest,
    }
    if shared:
        roofline["logical_bytes_per_launch"] = logical
        roofline["logical_gbps"] = round(logical / (main_ms * 1e-3) / 1e9, 1)

    def dist(ms):
        med = float(np.median(ms))
        return {"median_us": round(med * 1e3, 2), "p10_us": round(float(np.percentile(ms, 10)) * 1e3, 2),
                "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 2), "mean_us": round(float(np.mean(ms)) * 1e3, 2),
                "gbps_median": round(kv_bytes / (med * 1e-3) / 1e9, 1),
                "frac_median": round(kv_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    rec = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "decode_seqs_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "config": {
            "workload": w.name, "description": w.description, "num_seqs": w.num_seqs,
            "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "sum_context_tokens": int(w.context_lens.sum()),
            "max_context_len": w.max_context_len, "num_blocks": w.num_blocks,
            "partition_size": P, "kernel": main_name if prefix else kernel_name, "reuse": reuse,
            "seed": w.seed, "shared_len": shared_len,
            "kv_bytes_per_step": kv_bytes, "logical_kv_bytes_per_step": logical,
            "appended_tokens_per_step": int((slots >= 0).sum()), "step": a.step,
        },
        "step_event_us": round(step_event_ms * 1e3, 2),
        "kernels_avg_us": {
            "kv_append": round(append_ms * 1e3, 2) if append_ms is not None else None,
            main_name: round(main_ms * 1e3, 2),
            "decode_reduce": round(reduce_ms * 1e3, 2) if reduce_ms is not None else None,
        },
        "step_timing": {"warm": dist(warm), "cold": dist(cold), "samples": nsamp,
                        "cold_eviction": "1 GiB write + 1 GiB read before each step, outside the events"},
        "roofline": roofline,
    }
    if shared:
        rec["logical_kv_gbps"] = round(logical / (ms_per_step * 1e-3) / 1e9, 1)
    # achievable read bandwidth on this device: a plain streaming read of
    # 2 GiB, and of exactly the bytes one decode step reads
    rec["stream_read_reference_gbps"] = {
        "2GiB": stream_read_gbps(torch, pa, 2 << 30),
        "step_bytes": stream_read_gbps(torch, pa, kv_bytes),
    }
    rec["roofline"]["frac_of_stream_read"] = round(
        achieved / rec["stream_read_reference_gbps"]["step_bytes"], 4)
    if not a.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, t, a.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def _loop_ms(torch, stream, fn, n):
    """Average ms per call of `n` back-to-back calls of `fn`, from one event
    pair on `stream` around them."""
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _step_samples(torch, stream, fn, n, before=None):
    """Milliseconds of each of `n` calls of `fn`, each between its own event
    pair on `stream`; `before` (if given) runs ahead of each pair."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for s0, s1 in evs:
        if before is not None:
            before()
        s0.record(stream)
        fn()
        s1.record(stream)
    torch.cuda.synchronize()
    return [s0.elapsed_time(s1) for s0, s1 in evs]


class _Evictor:
    """Evicts L2 and the Infinity Cache: writes one buffer of `nbytes` and
    reads another (ordinary cached loads), so the caches end up holding
    neither the step's pages nor dirty lines."""

    def __init__(self, torch, pa, nbytes):
        self.pa = pa
        self.w = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
        self.r = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.k = 0

    def __call__(self):
        self.k ^= 1
        self.w.fill_(self.k)
        self.pa.probe_stream_read(self.r, self.sink, nontemporal=False)


if __name__ == "__main__":
    sys.exit(main())
