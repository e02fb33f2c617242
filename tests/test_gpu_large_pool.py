"""A pool far past 4 GiB per cache (300,000 pages of 32 KiB: about 9.8 GB for
K and as much for V), with the sequences' pages at the top of it, so every
byte offset the kernels form for those pages exceeds 32 bits.  Append, page
copy, decode (one pass and split) and multi-query attention run on it.

The oracle works on a small host pool holding only the pages in use,
renumbered 0 .. n-1, filled by its own append and copy of the same rows; no
oracle input comes from the device."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_close, out_f64, require_gpu, say, storage_np

pytestmark = pytest.mark.gpu

NB, BS, HQ, HKV, D = 300_000, 16, 32, 8, 128


def test_pool_beyond_four_gib():
    pa = require_gpu()
    if torch.cuda.get_device_properties(0).total_memory < 64 * (1 << 30):
        pytest.skip("needs a device with room for two 9.8 GB caches")
    rng = np.random.default_rng(51)
    lens = [1000, 2500, 700, 3000]
    npg = [-(-L // BS) for L in lens]
    # pages drawn from the top of the pool, plus the very last page
    top = rng.choice(np.arange(NB - 60_000, NB - 1), size=sum(npg) + 1, replace=False).tolist()
    pages = [NB - 1] + top
    tables = np.full((len(lens), max(npg)), pages[-1], dtype=np.int32)
    at = 0
    for b, n in enumerate(npg):
        tables[b, :n] = pages[at:at + n]
        at += n
    spare = pages[at]                                   # copy-on-write target
    assert (tables[:, 0] > 2 ** 32 // (HKV * D * BS * 2)).any()       # offsets past 4 GiB

    say("large pool: allocating", NB, "pages per cache")
    kc = torch.empty((NB, HKV, D // 8, BS, 8), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty((NB, HKV, D, BS), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cpu")
    g.manual_seed(52)
    T = sum(lens)
    k = torch.randn(T, HKV, D, generator=g).to(torch.bfloat16)
    v = torch.randn(T, HKV, D, generator=g).to(torch.bfloat16)
    slots = np.concatenate([tables[b][np.arange(L) // BS].astype(np.int64) * BS + np.arange(L) % BS
                            for b, L in enumerate(lens)])
    pa.kv_append(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), kc, vc)
    # copy-on-write of sequence 0's last page to the spare page, then point the table at it
    last = int(tables[0, npg[0] - 1])
    pa.copy_blocks(kc, vc, torch.tensor([[last, spare]], dtype=torch.int64, device="cuda"))
    tables[0, npg[0] - 1] = spare

    # oracle pool: the pages in use renumbered, filled by the oracle's own append and copy
    used = sorted(set(pages))
    where = {p: i for i, p in enumerate(used)}
    hk = np.zeros((len(used), HKV, D // 8, BS, 8), dtype=np.uint16)
    hv = np.zeros((len(used), HKV, D, BS), dtype=np.uint16)
    hslots = np.array([where[int(s // BS)] * BS + int(s % BS) for s in slots], dtype=np.int64)
    hk, hv = oracle.kv_append(storage_np(k), storage_np(v), hslots, hk, hv, BS)
    hk, hv = oracle.copy_blocks(hk, hv, np.array([[where[last], where[spare]]], dtype=np.int64))
    htab = np.vectorize(lambda p: where[int(p)])(tables).astype(np.int32)
    hlens = np.array(lens, dtype=np.int32)

    q = torch.randn(len(lens), HQ, D, generator=g).to(torch.bfloat16)
    scale = float(np.float32(1 / np.sqrt(D)))
    ref = oracle.decode(storage_np(q), hk, hv, htab, hlens, scale, BS, "bf16")
    bt, cl = torch.from_numpy(tables).cuda(), torch.from_numpy(hlens).cuda()
    for P in (-1, 256):
        say("large pool decode, partition", P)
        out = pa.decode(q.cuda(), kc, vc, bt, cl, scale, max(lens), partition_size=P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"large pool decode P={P}")

    # multi-query: the last three tokens of each sequence as new tokens
    qs = np.arange(0, 3 * len(lens) + 1, 3, dtype=np.int32)
    qm = torch.randn(3 * len(lens), HQ, D, generator=g).to(torch.bfloat16)
    refm = oracle.decode_multi(storage_np(qm), hk, hv, htab, hlens, qs, scale, BS, "bf16")
    for P in (-1, 512):
        say("large pool multi-query, partition", P)
        outm = pa.decode_multi(qm.cuda(), kc, vc, bt, cl, torch.from_numpy(qs).cuda(), scale, max(lens), 3,
                               partition_size=P)
        torch.cuda.synchronize()
        check_close(out_f64(outm), refm, "bf16", f"large pool multi P={P}")
    del kc, vc
    torch.cuda.empty_cache()
