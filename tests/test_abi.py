"""The C-ABI library loads, exports every symbol include/*.h declares, and
rejects bad arguments on the host (CPU only: no call here reaches the GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

pa = pytest.importorskip("paged_kv_cache_350_amd")


def declared_functions():
    names = set()
    for header in HEADERS:
        text = open(header).read()
        names |= set(re.findall(r"^\s*(?:pa_status|size_t|int32_t|int64_t|void|const char\*)\s+(pa_\w+)\s*\(",
                                text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pa.LIB_PATH):
        pytest.fail("libpa.so is not built (python -m paged_kv_cache_350_amd.build)")
    return pa.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["pa_kv_append", "pa_decode", "pa_copy_blocks", "pa_decode_workspace_size",
                 "pa_status_string", "pa_decode_partition", "pa_decode_reduce",
                 "pa_decode_partition_size", "pa_version", "pa_probe_stream_read",
                 "pa_decode_append", "pa_decode_shared_prefix"]:
        assert want in names


def test_every_declared_symbol_is_exported(L):
    raw = ctypes.CDLL(pa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert pa.status_string(code)
    assert pa.status_string(0) == "ok"
    assert pa.status_string(-99) == "unknown status"
    assert L.pa_version() == 331


def test_partition_policy_and_workspace_size(L):
    # explicit sizes and single pass
    assert pa.decode_partition_size(64, 8, 4096, -1) == 0
    assert pa.decode_partition_size(64, 8, 4096, 256) == 256
    assert pa.decode_partition_size(64, 8, 4096, 100) < 0        # not a multiple of 32
    assert pa.decode_partition_size(64, 8, 4096, 16) < 0
    assert pa.decode_partition_size(64, 8, -1, 0) < 0
    # library default for streaming loads, worked through the rule in pa.h:
    assert pa.decode_partition_size(64, 8, 512, 0) == 0          # short: single pass
    assert pa.decode_partition_size(64, 8, 4027, 0) == 0         # 8B-shaped batch: 512 pairs, longest first
    assert pa.decode_partition_size(256, 8, 8192, 0) == 0        # 70B-shaped batch: 2,048 pairs, one pass
    assert pa.decode_partition_size(128, 8, 2048, 0) == 0        # 1,024 pairs, contexts <= 4,096: one pass
    assert pa.decode_partition_size(128, 8, 8192, 0) == 4096     # 1,024 pairs, longer contexts
    assert pa.decode_partition_size(8, 8, 32768, 0) == 2048      # long context: 4096 gives only 512 units
    assert pa.decode_partition_size(32, 8, 16384, 0) == 4096
    assert pa.decode_partition_size(512, 8, 32768, 0) == 0       # plenty of pairs
    assert pa.decode_partition_size(1, 8, 32768, 0) == 256       # one sequence: the shared-page rule
    assert pa.decode_partition_size(2, 1, 600, 0) == 256
    assert pa.decode_partition_size(64, 8, 4027, 0, "stream") == 0
    assert pa.decode_partition_size(64, 8, 16384, 0) == 8192     # 512 pairs, but contexts past 8,192
    assert pa.decode_partition_size(300, 2, 4027, 0) == 2048     # 600 pairs, but more than 256 sequences
    assert pa.decode_partition_size(63, 8, 4027, 0) == 2048      # 504 pairs: below the ordered one pass
    # shared pages: the longest partition with 4 per longest context and 1,024 workgroups
    assert pa.decode_partition_size(64, 8, 4027, 0, "shared") == 512
    assert pa.decode_partition_size(256, 8, 8192, 0, "shared") == 2048
    assert pa.decode_partition_size(100, 8, 10512, 0, "shared") == 2048    # prefix sharing
    assert pa.decode_partition_size(8, 8, 32774, 0, "shared") == 2048      # beams
    assert pa.decode_partition_size(512, 8, 32768, 0, "shared") == 4096
    assert pa.decode_partition_size(1, 8, 32768, 0, "shared") == 256
    assert L.pa_decode_partition_size(64, 8, 4027, 0, 7) < 0            # unknown load path
    assert L.pa_decode_workspace_size(64, 32, 8, 128, 4027, 0, 7) == 0
    # workspace = seqs x heads x parts x (D + 2) floats
    assert pa.decode_workspace_size(8, 32, 8, 128, 32768, 512) == 8 * 32 * 64 * 130 * 4
    assert pa.decode_workspace_size(64, 32, 8, 128, 4096, 0) == 0                       # one pass
    assert pa.decode_workspace_size(63, 32, 8, 128, 4096, 0) == 63 * 32 * 2 * 130 * 4   # P = 2048 at 4,096
    assert pa.decode_workspace_size(64, 32, 8, 128, 4096, 0, "shared") == 64 * 32 * 4 * 130 * 4   # P = 1024
    assert pa.decode_workspace_size(256, 64, 8, 128, 8192, 0) == 0                      # one pass
    assert pa.decode_workspace_size(256, 64, 8, 128, 8192, 0, "shared") == 256 * 64 * 4 * 130 * 4
    assert pa.decode_workspace_size(64, 32, 8, 128, 500, 0) == 0
    assert pa.decode_workspace_size(64, 32, 8, 128, 4096, -1) == 0
    assert pa.decode_workspace_size(3, 4, 4, 64, 33, 32) == 3 * 4 * 2 * 66 * 4
    assert pa.decode_workspace_size(3, 4, 0, 64, 33, 32) == 0


FAKE = 1 << 20          # 16-byte aligned, never dereferenced: validation fails first


def _decode(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, bs=16, hkv=8, scale=0.1, out=FAKE,
             stream=None, B=4, hq=32, d=128, maxb=16, maxctx=256, nb=100, dtype=1, part=0,
             kernel=0, reuse=0, ws=None, wsb=0)
    a.update(kw)
    return L.pa_decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["bs"], a["hkv"], a["scale"],
                       a["out"], a["stream"], a["B"], a["hq"], a["d"], a["maxb"], a["maxctx"],
                       a["nb"], a["dtype"], a["part"], a["kernel"], a["reuse"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), pa.PA_ERR_NULL),
    (dict(out=None), pa.PA_ERR_NULL),
    (dict(bt=None), pa.PA_ERR_NULL),
    (dict(bs=8), pa.PA_ERR_UNSUPPORTED),
    (dict(d=96), pa.PA_ERR_UNSUPPORTED),
    (dict(hq=30), pa.PA_ERR_ARG),                     # not a multiple of kv heads
    (dict(hq=136, hkv=8), pa.PA_ERR_UNSUPPORTED),     # 17 query heads per kv head
    (dict(hkv=0), pa.PA_ERR_ARG),
    (dict(dtype=7), pa.PA_ERR_ARG),
    (dict(kernel=9), pa.PA_ERR_ARG),
    (dict(reuse=3), pa.PA_ERR_ARG),
    (dict(reuse=-1), pa.PA_ERR_ARG),
    (dict(dtype=0, kernel=2), pa.PA_ERR_UNSUPPORTED), # MFMA kernel is bf16 only
    (dict(maxctx=257), pa.PA_ERR_ARG),                # beyond max_blocks_per_seq * block_size
    (dict(maxctx=-1), pa.PA_ERR_ARG),
    (dict(nb=0), pa.PA_ERR_ARG),
    (dict(part=48), pa.PA_ERR_ARG),
    (dict(part=256), pa.PA_ERR_WORKSPACE),            # split path without workspace
    (dict(part=256, ws=FAKE, wsb=16), pa.PA_ERR_WORKSPACE),
    (dict(q=FAKE + 4), pa.PA_ERR_ARG),                # misaligned
    (dict(scale=float("nan")), pa.PA_ERR_ARG),
    (dict(B=-1), pa.PA_ERR_ARG),
])
def test_decode_rejects_bad_arguments(L, kw, status):
    assert _decode(L, **kw) == status


def test_zero_sequences_is_a_no_op(L):
    assert _decode(L, B=0, q=None, out=None, bt=None, cl=None) == pa.PA_OK


def test_stage_entry_points_validate(L):
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 16, 8, 0.1, None, 4, 32, 128, 16, 256, 100, 1]
    N = (None, None, None)                 # no fused append
    assert L.pa_decode_partition(*args, 0, 0, 0, FAKE, 1 << 30, *N) == pa.PA_ERR_ARG   # needs explicit P
    assert L.pa_decode_partition(*args, -1, 0, 0, FAKE, 1 << 30, *N) == pa.PA_ERR_ARG
    assert L.pa_decode_partition(*args, 64, 0, 0, None, 0, *N) == pa.PA_ERR_WORKSPACE
    assert L.pa_decode_partition(*args, 64, 0, 5, FAKE, 1 << 30, *N) == pa.PA_ERR_ARG  # bad reuse
    # a fused append needs both rows, 16-byte aligned
    assert L.pa_decode_partition(*args, 64, 0, 0, FAKE, 1 << 30, FAKE, None, None) == pa.PA_ERR_NULL
    assert L.pa_decode_partition(*args, 64, 0, 0, FAKE, 1 << 30, FAKE, FAKE + 2, None) == pa.PA_ERR_ARG
    assert L.pa_decode_reduce(FAKE, 16, FAKE, FAKE, None, 4, 32, 128, 256, 64, 1) == pa.PA_ERR_WORKSPACE
    assert L.pa_decode_reduce(FAKE, 1 << 30, FAKE, FAKE, None, 4, 32, 128, 256, 0, 1) == pa.PA_ERR_ARG
    assert L.pa_decode_reduce(FAKE, 1 << 30, None, FAKE, None, 4, 32, 128, 256, 64, 1) == pa.PA_ERR_NULL
    assert L.pa_decode_reduce(FAKE, 1 << 30, FAKE, FAKE, None, 4, 32, 96, 256, 64, 1) == pa.PA_ERR_UNSUPPORTED


def test_append_and_copy_validate(L):
    # pa_kv_append(k, v, slots, kc, vc, T, hkv, d, bs, nb, dtype, stream)
    assert L.pa_kv_append(None, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 1, None) == pa.PA_ERR_NULL
    assert L.pa_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 24, 10, 1, None) == pa.PA_ERR_UNSUPPORTED
    assert L.pa_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 10, 1, None) == pa.PA_ERR_ARG
    assert L.pa_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 0, 1, None) == pa.PA_ERR_ARG
    assert L.pa_kv_append(FAKE + 2, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 1, None) == pa.PA_ERR_ARG
    assert L.pa_kv_append(None, None, None, None, None, 0, 8, 128, 16, 10, 1, None) == pa.PA_OK
    # pa_copy_blocks(kc, vc, mapping, n, hkv, d, bs, nb, dtype, stream)
    assert L.pa_copy_blocks(FAKE, FAKE, None, 3, 8, 128, 32, 10, 1, None) == pa.PA_ERR_NULL
    assert L.pa_copy_blocks(FAKE, FAKE, FAKE, 3, 8, 64, 12, 10, 1, None) == pa.PA_ERR_UNSUPPORTED
    assert L.pa_copy_blocks(FAKE, FAKE, FAKE, -3, 8, 64, 16, 10, 1, None) == pa.PA_ERR_ARG
    assert L.pa_copy_blocks(FAKE, FAKE, FAKE, 3, 8, 64, 16, 10, 5, None) == pa.PA_ERR_ARG
    assert L.pa_copy_blocks(None, None, None, 0, 8, 64, 16, 10, 1, None) == pa.PA_OK


def test_binding_refuses_cpu_tensors():
    import torch
    kc = torch.zeros(4, 2, 16, 16, 8, dtype=torch.bfloat16)
    vc = torch.zeros(4, 2, 128, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        pa.copy_blocks(kc, vc, torch.zeros(1, 2, dtype=torch.int64))


def test_probe_validates(L):
    # pa_probe_stream_read(buf, bytes, nontemporal, num_workgroups, sink, stream)
    assert L.pa_probe_stream_read(FAKE, 100, 1, 0, FAKE, None) == pa.PA_ERR_ARG      # not 16-byte multiple
    assert L.pa_probe_stream_read(FAKE, 1024, 2, 0, FAKE, None) == pa.PA_ERR_ARG
    assert L.pa_probe_stream_read(None, 1024, 1, 0, FAKE, None) == pa.PA_ERR_NULL
    assert L.pa_probe_stream_read(FAKE + 8, 1024, 1, 0, FAKE, None) == pa.PA_ERR_ARG
    assert L.pa_probe_stream_read(None, 0, 1, 0, None, None) == pa.PA_OK


def test_decode_append_validates(L):
    # pa_decode_append(k_new, v_new, slot_mapping, q, kc, vc, bt, cl, bs, hkv, scale, out, stream,
    #                  B, hq, d, maxb, maxctx, nb, dtype, part, kernel, reuse, ws, wsb)
    def call(**kw):
        a = dict(kn=FAKE, vn=FAKE, sm=None, q=FAKE, B=4, bs=16, ws=None, wsb=0, part=-1, reuse=0)
        a.update(kw)
        return L.pa_decode_append(a["kn"], a["vn"], a["sm"], a["q"], FAKE, FAKE, FAKE, FAKE, a["bs"], 8,
                                  0.1, FAKE, None, a["B"], 32, 128, 16, 256, 100, 1, a["part"], 0,
                                  a["reuse"], a["ws"], a["wsb"])
    assert call(kn=None) == pa.PA_ERR_NULL
    assert call(vn=None) == pa.PA_ERR_NULL
    assert call(kn=FAKE + 8) == pa.PA_ERR_ARG
    assert call(q=None) == pa.PA_ERR_NULL
    assert call(bs=8) == pa.PA_ERR_UNSUPPORTED
    assert call(reuse=7) == pa.PA_ERR_ARG
    assert call(part=256) == pa.PA_ERR_WORKSPACE
    assert call(B=0, kn=None, vn=None, q=None) == pa.PA_OK


def test_decode_multi_validates(L):
    """pa_decode_multi argument checks (all fail on the host, before any launch)."""
    def call(**kw):
        a = dict(q=FAKE, qs=FAKE, out=FAKE, B=4, T=20, hq=32, hkv=8, d=128, maxb=256, ctx=4096,
                 maxq=5, dtype=1, part=0, reuse=0, ws=FAKE, wsb=1 << 30, bs=16, scale=0.1)
        a.update(kw)
        return L.pa_decode_multi(a["q"], FAKE, FAKE, FAKE, FAKE, a["qs"], a["bs"], a["hkv"], a["scale"],
                                 a["out"], None, a["B"], a["T"], a["hq"], a["d"], a["maxb"], a["ctx"],
                                 a["maxq"], 100000, a["dtype"], a["part"], a["reuse"], a["ws"], a["wsb"])
    assert call(B=0) == pa.PA_OK and call(T=0) == pa.PA_OK          # nothing to do
    assert call(dtype=0) == pa.PA_ERR_UNSUPPORTED                    # fp32: no multi-query kernel
    assert call(dtype=7) == pa.PA_ERR_ARG
    assert call(maxq=0) == pa.PA_ERR_ARG
    assert call(maxq=1025) == pa.PA_ERR_UNSUPPORTED
    assert call(qs=None) == pa.PA_ERR_NULL
    assert call(out=None) == pa.PA_ERR_NULL
    assert call(q=FAKE + 2) == pa.PA_ERR_ARG
    assert call(ws=None, part=256) == pa.PA_ERR_WORKSPACE            # split path needs a workspace
    assert call(wsb=16, part=256) == pa.PA_ERR_WORKSPACE
    assert call(hq=24, hkv=8, d=96) == pa.PA_ERR_UNSUPPORTED
    assert call(hq=30) == pa.PA_ERR_ARG                              # not a multiple of kv heads
    assert call(part=100) == pa.PA_ERR_ARG
    assert call(reuse=9) == pa.PA_ERR_ARG
    assert call(ctx=4097) == pa.PA_ERR_ARG                            # beyond the table width
    assert call(scale=float("nan")) == pa.PA_ERR_ARG
    assert call(B=-1) == pa.PA_ERR_ARG


def test_decode_multi_partition_policy(L):
    f = pa.decode_multi_partition_size
    # explicit sizes behave as for pa_decode
    assert f(64, 32, 8, 4096, 5, -1) == 0 and f(64, 32, 8, 4096, 5, 256) == 256
    assert f(64, 32, 8, 4096, 5, 100) < 0 and f(64, 32, 8, 4096, 0, 0) < 0
    # default: one pass once (sequence, column group, kv head) units fill the chip (>= 256)
    assert f(64, 32, 8, 4096, 5, 0) == 0          # 64 x 1 x 8 = 512 units
    assert f(64, 32, 8, 512, 5, 0) == 0           # short contexts: one pass
    assert f(16, 32, 8, 4094, 5, 0) == 2048       # 128 units: two partitions each
    assert f(4, 32, 8, 8192, 8, 0) == 1024        # 32 units x 8 partitions
    assert f(8, 32, 8, 32768, 5, 0) == 8192       # long contexts: 64 units x 4
    assert f(2, 32, 8, 600, 5, 0) == 256          # nothing fills the chip: the shortest partition
    # from 64 columns (4 x 16) the LDS-staged kernel: one 128-column group, 128 units, four partitions
    # reach its fill of 512 workgroups
    assert f(16, 32, 8, 4094, 16, 0) == 1024
    assert f(64, 32, 8, 4096, 16, 0) == 0         # 512 units: one pass
    assert f(8, 32, 8, 4096, 512, 0) == 0         # a prompt chunk: 16 column groups, 1,024 units
    # workspace rows are query tokens
    want = 320 * 32 * (-(-4096 // 256)) * (128 + 2) * 4
    assert pa.decode_multi_workspace_size(64, 320, 32, 8, 128, 4096, 5, 256) == want
    assert pa.decode_multi_workspace_size(64, 320, 32, 8, 128, 4096, 5, 0) == 0


def test_decode_multi_append_validates(L):
    def call(kn=FAKE, vn=FAKE, **kw):
        a = dict(q=FAKE, B=4, T=20, maxq=5, part=0)
        a.update(kw)
        return L.pa_decode_multi_append(kn, vn, a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, 16, 8, 0.1, FAKE, None,
                                        a["B"], a["T"], 32, 128, 256, 4096, a["maxq"], 100000, 1, a["part"], 0,
                                        FAKE, 1 << 30)
    assert call(kn=None) == pa.PA_ERR_NULL
    assert call(vn=None) == pa.PA_ERR_NULL
    assert call(kn=FAKE + 2) == pa.PA_ERR_ARG
    assert call(kn=None, vn=None, B=0) == pa.PA_OK          # nothing to do
    assert call(maxq=0) == pa.PA_ERR_ARG


def _shared(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, bs=16, hkv=8, scale=0.1, out=FAKE,
             stream=None, B=4, hq=32, d=128, maxb=16, maxctx=256, nb=100, dtype=1, S=128, part=64,
             ws=FAKE, wsb=1 << 30, kn=None, vn=None, sm=None)
    a.update(kw)
    return L.pa_decode_shared_prefix(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["bs"], a["hkv"], a["scale"],
                                     a["out"], a["stream"], a["B"], a["hq"], a["d"], a["maxb"], a["maxctx"],
                                     a["nb"], a["dtype"], a["S"], a["part"], a["ws"], a["wsb"],
                                     a["kn"], a["vn"], a["sm"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), pa.PA_ERR_UNSUPPORTED),           # matrix-core kernels: bf16 only
    (dict(dtype=5), pa.PA_ERR_ARG),
    (dict(B=1025), pa.PA_ERR_UNSUPPORTED),            # prefix launch rows
    (dict(part=-32), pa.PA_ERR_ARG),
    (dict(part=48), pa.PA_ERR_ARG),
    (dict(S=100), pa.PA_ERR_ARG),                     # not whole pages
    (dict(S=-64), pa.PA_ERR_ARG),
    (dict(S=320), pa.PA_ERR_ARG),                     # beyond max_context_len
    (dict(ws=None, wsb=0), pa.PA_ERR_WORKSPACE),
    (dict(wsb=16), pa.PA_ERR_WORKSPACE),
    (dict(S=144, wsb=4 * 32 * 4 * 130 * 4), pa.PA_ERR_WORKSPACE),   # the split path's size: a slot short
    (dict(q=None), pa.PA_ERR_NULL),
    (dict(bs=8), pa.PA_ERR_UNSUPPORTED),
    (dict(B=0), pa.PA_OK),                            # nothing to do, nothing launched
    (dict(kn=FAKE), pa.PA_ERR_NULL),                  # K rows without V rows
    (dict(kn=FAKE, vn=FAKE + 8), pa.PA_ERR_ARG),      # misaligned
])
def test_decode_shared_prefix_validates(L, kw, status):
    assert _shared(L, **kw) == status


def test_shared_prefix_len_from_tables():
    t = np.array([[1, 2, 3, 4], [1, 2, 5, 6], [1, 2, 3, 7]])
    assert pa.shared_prefix_len(t, np.array([60, 50, 64]), 16) == 32
    assert pa.shared_prefix_len(t, np.array([60, 20, 64]), 16) == 16      # shortest context caps it, whole pages
    assert pa.shared_prefix_len(t[:1], np.array([60]), 16) == 48
    assert pa.shared_prefix_len(t[:, :0], np.array([5, 5, 5]), 16) == 0
    assert pa.shared_prefix_len(t, np.array([], dtype=np.int32), 16) == 0


def test_shared_prefix_workspace_size():
    # the prefix launch's partitions first, then the per-sequence ones from
    # shared_len / P on; with the prefix launch at partition P that is the
    # split path's row plus one slot when shared_len ends inside a partition
    assert pa.shared_prefix_workspace_size(3, 4, 4, 64, 33, 0, 32) == 3 * 4 * 2 * 66 * 4
    assert pa.shared_prefix_workspace_size(3, 4, 4, 64, 96, 64, 32) == 3 * 4 * 3 * 66 * 4
    assert pa.shared_prefix_workspace_size(3, 4, 4, 64, 96, 48, 32) == 3 * 4 * 4 * 66 * 4
    assert pa.shared_prefix_workspace_size(3, 4, 4, 64, 33, 0, 48) == 0                  # not a multiple of 32
    assert pa.shared_prefix_workspace_size(3, 4, 4, 64, 33, 40, 32) == 0                 # past max_context_len
    assert pa.shared_prefix_workspace_size(-1, 4, 4, 64, 33, 0, 32) == 0
    # 100 sequences x 4 query heads per kv head = 400 columns: the LDS-staged
    # prefix stage on 4-wave workgroups, 4 column groups of 128 x 8 kv heads
    # = 32 workgroups per partition, so 8 partitions for about 1,024 waves,
    # of ceil(9984 / 8) = 1248 tokens rounded up to the 64-token chunk = 1280:
    # 8 prefix slots, then the per-sequence partitions 4 and 5 of the
    # default 2048 -> 10 slots per row
    assert pa.shared_prefix_workspace_size(100, 32, 8, 128, 10512, 9984, 0) == \
        pa.shared_prefix_workspace_size(100, 32, 8, 128, 10512, 9984, 2048) == 100 * 32 * 10 * 130 * 4
    # 24 sequences x 4 = 96 columns, one 4-wave column group: 8 workgroups per
    # partition would ask for 64 partitions, but they are at least 4 chunks
    # (256 tokens): 3 prefix slots; the per-sequence partitions of 32 start
    # at 640 / 32 = 20, shifted to slot 3 -> ceil(1036 / 32) - 20 + 3 = 16
    assert pa.shared_prefix_workspace_size(24, 32, 8, 128, 1036, 640, 32) == 24 * 32 * 16 * 130 * 4


def _groups(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, bs=16, hkv=8, scale=0.1, out=FAKE,
             stream=None, B=4, hq=32, d=128, maxb=16, maxctx=256, nb=100, dtype=1, G=2, gs=FAKE, gl=FAKE,
             sl=FAKE, maxg=3, maxs=128, part=64, ws=FAKE, wsb=1 << 30, kn=None, vn=None, sm=None)
    a.update(kw)
    return L.pa_decode_shared_prefix_groups(
        a["q"], a["k"], a["v"], a["bt"], a["cl"], a["bs"], a["hkv"], a["scale"], a["out"], a["stream"], a["B"],
        a["hq"], a["d"], a["maxb"], a["maxctx"], a["nb"], a["dtype"], a["G"], a["gs"], a["gl"], a["sl"],
        a["maxg"], a["maxs"], a["part"], a["ws"], a["wsb"], a["kn"], a["vn"], a["sm"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), pa.PA_ERR_UNSUPPORTED),
    (dict(G=-1), pa.PA_ERR_ARG),
    (dict(maxg=0), pa.PA_ERR_ARG),
    (dict(maxg=1025), pa.PA_ERR_UNSUPPORTED),
    (dict(maxs=-1), pa.PA_ERR_ARG),
    (dict(maxs=512), pa.PA_ERR_ARG),                  # beyond max_context_len
    (dict(part=48), pa.PA_ERR_ARG),
    (dict(sl=None), pa.PA_ERR_NULL),
    (dict(gs=None), pa.PA_ERR_NULL),
    (dict(gl=None), pa.PA_ERR_NULL),
    (dict(kn=FAKE), pa.PA_ERR_NULL),
    (dict(ws=None, wsb=0), pa.PA_ERR_WORKSPACE),
    (dict(wsb=4 * 32 * 4 * 130 * 4), pa.PA_ERR_WORKSPACE),   # the split path's size: a slot short
    (dict(B=0), pa.PA_OK),
])
def test_decode_shared_prefix_groups_validates(L, kw, status):
    assert _groups(L, **kw) == status


def test_shared_prefix_groups_workspace_size(L):
    assert L.pa_decode_shared_prefix_groups_workspace_size(4, 32, 128, 256, 64) == 4 * 32 * 5 * 130 * 4
    # the split row (ceil(10512 / 2048) = 6) plus the prefix slots an LDS-staged
    # prefix launch may write, partitions of at least 256 tokens: ceil(10512 / 256) = 42
    assert L.pa_decode_shared_prefix_groups_workspace_size(4, 32, 128, 10512, 0) == 4 * 32 * 48 * 130 * 4
    assert L.pa_decode_shared_prefix_groups_workspace_size(4, 32, 128, 256, 48) == 0
