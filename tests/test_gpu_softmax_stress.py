"""Score patterns that stress the online softmax, on the GPU.

The query is one-hot on dim 0 and K[t][h][0] = s_t / scale, so the scores are
exactly the pattern s_t (up to the storage rounding of K, which the oracle
sees too):

* ramp up     -- the maximum grows by 16 every 32-token chunk, so the
                 running reference moves on nearly every chunk;
* ramp down   -- the first chunk holds the maximum, later weights underflow;
* late spike  -- one token near the end 200 above everything else;
* sawtooth    -- +-30 swings with a period of 44 tokens;
* flat        -- every score equal: the output is the mean of V.

Tolerances: bf16 as everywhere.  fp32 scores of magnitude S are themselves
rounded by the device (the oracle works in float64): one rounding of a score
in log2 units moves its weight by up to 2^-24 * S * log2(e) * ln(2) = 2^-24 * S
relative, so the output may move by twice that times max|V|.  The fp32 bound
is therefore 1e-5 + 2^-23 * S_max * max|V|: 1e-5 for the flat pattern, about
5.5e-4 for the ramp whose scores reach 1,024.

Both decode kernels run single pass and with small partitions (so the merge
sees partials whose maxima differ by hundreds), and the multi-query kernel
runs on the same caches.  Caches are built on the host and uploaded with a
plain copy: the oracle never reads anything the library wrote."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_close, out_f64, require_gpu, say, storage_np

pytestmark = pytest.mark.gpu

LENS = [700, 2049, 33, 96]
HQ, HKV, D, BS = 8, 2, 128, 16


def pattern(name, L, rng):
    t = np.arange(L, dtype=np.float64)
    if name == "ramp_up":
        return 0.5 * t
    if name == "ramp_down":
        return -0.5 * t
    if name == "late_spike":
        s = rng.standard_normal(L)
        s[max(L - 3, 0)] += 200.0
        return s
    if name == "sawtooth":
        return 30.0 * np.sin(t / 7.0)
    if name == "flat":
        return np.zeros(L)
    raise ValueError(name)


def build(name, dtype):
    """Host caches (storage form), tables, lengths, q and scale for a pattern."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    x = 16 // (4 if dtype == "f32" else 2)
    scale = float(np.float32(1 / np.sqrt(D)))
    npg = [-(-L // BS) for L in LENS]
    nb = sum(npg) + 2
    perm = rng.permutation(nb)
    tables = np.full((len(LENS), max(npg)), perm[-1], dtype=np.int32)
    kc = torch.full((nb, HKV, D // x, BS, x), float("nan"), dtype=td)
    vc = torch.full((nb, HKV, D, BS), float("nan"), dtype=td)
    at = 0
    for b, L in enumerate(LENS):
        pages = perm[at:at + npg[b]]
        at += npg[b]
        tables[b, :npg[b]] = pages
        K = 0.05 * torch.from_numpy(rng.standard_normal((L, HKV, D))).float()
        K[:, :, 0] = torch.from_numpy(pattern(name, L, rng) / scale).float()[:, None]
        V = torch.from_numpy(rng.standard_normal((L, HKV, D))).float()
        K, V = K.to(td), V.to(td)
        pos = torch.arange(L)
        pg = torch.from_numpy(pages.astype(np.int64))[pos // BS]
        off = pos % BS
        for h in range(HKV):
            kc[pg, h, :, off, :] = K[:, h, :].reshape(L, D // x, x)
            vc[pg, h, :, off] = V[:, h, :]
    q = torch.zeros(len(LENS), HQ, D)
    q[:, :, 0] = 1.0
    return kc.to(td), vc.to(td), tables, np.array(LENS, dtype=np.int32), q.to(td), scale


def f32_bound(name, vc):
    """1e-5 plus the effect of the device's fp32 rounding of the largest score."""
    if name == "late_spike":
        smax = 210.0                             # the spike plus the normal scores around it
    else:
        smax = max(float(np.abs(pattern(name, L, None)).max()) for L in LENS)
    vmax = float(np.nanmax(np.abs(vc.float().numpy())))
    return 1e-5 + 2.0 ** -23 * smax * vmax


@pytest.mark.parametrize("name", ["ramp_up", "ramp_down", "late_spike", "sawtooth", "flat"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_under_score_extremes(name, dtype):
    pa = require_gpu()
    kc, vc, tables, lens, q, scale = build(name, dtype)
    ref = oracle.decode(storage_np(q), storage_np(kc), storage_np(vc), tables, lens, scale, BS, dtype)
    kd, vd = kc.cuda(), vc.cuda()
    bt, cl, qd = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), q.cuda()
    for kernel in (["mfma", "valu"] if dtype == "bf16" else ["valu"]):
        for P in (-1, 64, 256):
            say("softmax stress", name, dtype, kernel, "partition", P)
            out = pa.decode(qd, kd, vd, bt, cl, scale, int(lens.max()), partition_size=P, kernel=kernel)
            torch.cuda.synchronize()
            check_close(out_f64(out), ref, dtype, f"{name} {dtype} {kernel} P={P}", f32_max_abs=f32_bound(name, vc))


@pytest.mark.parametrize("name", ["ramp_up", "late_spike", "sawtooth"])
def test_multi_query_under_score_extremes(name):
    """The last three tokens of each sequence as new tokens: columns whose
    visible prefixes end before the spike or the ramp's top."""
    pa = require_gpu()
    kc, vc, tables, lens, _, scale = build(name, "bf16")
    qs = np.arange(0, 3 * len(LENS) + 1, 3, dtype=np.int32)
    qm = torch.zeros(3 * len(LENS), HQ, D)
    qm[:, :, 0] = 1.0
    qm[1::3, :, 0] = 0.5                         # a second scale of scores among the columns
    qm = qm.to(torch.bfloat16)
    ref = oracle.decode_multi(storage_np(qm), storage_np(kc), storage_np(vc), tables, lens, qs, scale, BS, "bf16")
    for P in (-1, 64):
        say("multi softmax stress", name, "partition", P)
        out = pa.decode_multi(qm.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(tables).cuda(),
                              torch.from_numpy(lens).cuda(), torch.from_numpy(qs).cuda(), scale, int(lens.max()), 3,
                              partition_size=P)
        torch.cuda.synchronize()
        check_close(out_f64(out), ref, "bf16", f"multi {name} P={P}")
