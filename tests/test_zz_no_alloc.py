"""pa_decode_noalloc: pa_decode with the split path's partials in the
library's static per-GPU scratch instead of a caller workspace.

Each call is checked bit for bit against pa_decode with a workspace of
pa_decode_workspace_size() bytes (same kernels, same partitions), and
within the attention tolerances against the float64 oracle.  Two calls in a
row, the second smaller, show that what the first left in the scratch does
not leak into the second; a request larger than the scratch is refused on
the host with PA_ERR_SCRATCH and launches nothing."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import bits_equal, check_close, out_f64, require_gpu, say, step_and_reference

pytestmark = pytest.mark.gpu


def _both(pa, w, t, partition_size, kernel="auto"):
    """(noalloc output, pa_decode output) for the same request."""
    ws = pa.make_workspace(t["q"], w.num_kv_heads, w.max_context_len, partition_size)
    ref_out = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"], w.scale,
                        w.max_context_len, partition_size=partition_size, kernel=kernel, workspace=ws)
    out = torch.full_like(t["q"], float("nan"))
    pa.decode_noalloc(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"], w.scale,
                      w.max_context_len, out, partition_size=partition_size, kernel=kernel)
    torch.cuda.synchronize()
    return out, ref_out, ws


def test_two_calls_in_a_row_second_smaller():
    pa = require_gpu()
    cases = [
        # (workload, partition_size, kernel): the first fills more of the scratch than the second reads
        (W.custom("noalloc_big", 41, "bf16", [9000, 1, 4100, 6500, 33, 8191], 32, 8, 128, 16), 512, "auto"),
        (W.custom("noalloc_small", 42, "bf16", [700, 2000, 64], 32, 8, 128, 16), 256, "auto"),
    ]
    for w, ps, kernel in cases:
        need = pa.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                        w.max_context_len, ps)
        assert 0 < need <= pa.STATIC_SCRATCH_BYTES
        say("noalloc", w.name, w.summary(), "P", ps, "scratch bytes", need)
        t = W.make_tensors(w, "cuda")
        ref = step_and_reference(pa, w, t, range(w.num_seqs))
        out, ref_out, _ = _both(pa, w, t, ps, kernel)
        assert bits_equal(out, ref_out), f"{w.name}: noalloc differs from pa_decode"
        stats = check_close(out_f64(out), ref, w.dtype, f"noalloc {w.name}")
        say("  ", stats)


def test_fp32_vector_alu_and_single_pass():
    pa = require_gpu()
    w = W.custom("noalloc_f32", 43, "f32", [36, 42, 300, 129], 8, 2, 64, 16)
    say("noalloc", w.summary())
    t = W.make_tensors(w, "cuda")
    ref = step_and_reference(pa, w, t, range(w.num_seqs))
    for ps in (64, 32, -1):
        out, ref_out, _ = _both(pa, w, t, ps, "valu")
        assert bits_equal(out, ref_out), f"P={ps}: noalloc differs from pa_decode"
        check_close(out_f64(out), ref, "f32", f"noalloc f32 P={ps}")


def test_request_beyond_the_scratch_is_refused():
    pa = require_gpu()
    B, Hq, Hkv, D, bs, L = 256, 64, 8, 128, 16, 8192
    need = pa.decode_workspace_size(B, Hq, Hkv, D, L, 256)
    assert need > pa.STATIC_SCRATCH_BYTES
    say("noalloc refusal, workspace bytes", need)
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(4, Hkv, D // 8, bs, 8, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(4, Hkv, D, bs, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros(B, L // bs, dtype=torch.int32, device="cuda")
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 3.0)
    with pytest.raises(pa.PaError) as e:
        pa.decode_noalloc(q, kc, vc, tables, lens, 0.088, L, out, partition_size=256)
    assert e.value.status == pa.PA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call wrote its output"
