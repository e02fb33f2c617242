"""Build libpa.so (the C-ABI library) from csrc/*.hip with hipcc for gfx950.

    python -m paged_kv_cache_350_amd.build          # build in place
    python -m paged_kv_cache_350_amd.build --verbose

The library lands next to this file; the binding loads it from there.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
OBJDIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
# Packed fp32 VALU ops are switched off: the compiler would otherwise form
# v_pk_* float ops from ordinary float code.  MFMA results live in ordinary
# VGPRs (gfx950 has one unified register file): the decode kernel rescales
# its accumulators with vector ALU ops, which cannot read AGPRs, and in AGPR
# form the compiler copies them back and forth on every loop iteration.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpa)")


def sources():
    """HIP translation units (*.hip) and host-only C++ ones (*.cpp)."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool, extra) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return obj


def build(verbose: bool = False, extra=()) -> str:
    """Compile every csrc/*.hip and link libpa.so.  Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, list(extra)), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link of libpa.so failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel register / LDS / occupancy figures")
    args = ap.parse_args(argv)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if args.resource_usage else []
    build(verbose=args.verbose or args.resource_usage, extra=extra)
    return 0


if __name__ == "__main__":
    sys.exit(main())
