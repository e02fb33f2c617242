"""Turn rocprofv3 CSV output into the short summaries kept with the library.

Two summaries:

* ``stats`` -- per-kernel call count and average / min / max duration from a
  ``rocprofv3 --kernel-trace --stats --output-format csv`` run
  (``*_kernel_stats.csv``), for the kernels whose names contain the given
  substrings.
* ``counters`` -- the median per dispatch of every counter of one or more
  ``--pmc`` runs for one kernel (busy cycles, cache hits, instruction counts).
* ``traffic`` -- HBM bytes per launch of one kernel from two counter runs
  (``--pmc FETCH_SIZE``, then ``--pmc WRITE_SIZE``; both report KiB per
  dispatch), each scaled by what the same counter reads for a plain copy of
  known size.  The scale factors absorb whatever the counters do not see
  (on MI355X FETCH_SIZE reads about half of the bytes a copy kernel
  fetches, while WRITE_SIZE is exact).

    python -m paged_kv_cache_350_amd.profiling stats DIR --kernel decode_mfma ... \\
        --command "..." --out profiles/NAME.md
    python -m paged_kv_cache_350_amd.profiling traffic --fetch DIR --write DIR \\
        --calib-fetch DIR --calib-write DIR --kernel decode_mfma --calib-kernel copy_blocks \\
        --calib-bytes N [--calib-fetch-kernel stream_read_kernel<true> --calib-fetch-bytes N] \\
        --algorithmic-bytes N --source-digest HEX --out profiles/NAME.json
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys
from typing import Dict, List


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(run_dir: str, kernels: List[str]) -> List[Dict[str, object]]:
    path = _one(os.path.join(run_dir, "**", "*kernel_stats.csv"))
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if any(k in r["Name"] for k in kernels):
                rows.append({
                    "kernel": r["Name"].replace("(anonymous namespace)::", "").split("(")[0]
                              .replace("void ", ""),
                    "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3,
                    "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3,
                })
    return rows


def counter_per_dispatch(run_dir: str, kernel: str, counter: str) -> List[float]:
    """Values (KiB) of one counter for every dispatch of kernels matching ``kernel``."""
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError(f"no {counter} rows for kernel {kernel!r} in {path}")
    return vals


def traffic(fetch_dir: str, write_dir: str, calib_fetch_dir: str, calib_write_dir: str,
            kernel: str, calib_kernel: str, calib_bytes: int, calib_fetch_kernel: str = "",
            calib_fetch_bytes: int = 0) -> Dict[str, object]:
    """HBM bytes per launch of ``kernel``: FETCH_SIZE scaled by what it reads
    for a plain read of ``calib_fetch_bytes`` per dispatch (kernel
    ``calib_fetch_kernel``; default: the copy below), WRITE_SIZE by what it
    reads for a copy writing ``calib_bytes`` per dispatch (``calib_kernel``)."""
    fk = calib_fetch_kernel or calib_kernel
    fb = calib_fetch_bytes or calib_bytes
    kernels = kernel.split("+")           # several kernels of one call: the sum of their medians
    f_k = sum(statistics.median(counter_per_dispatch(fetch_dir, k, "FETCH_SIZE")) for k in kernels)
    w_k = sum(statistics.median(counter_per_dispatch(write_dir, k, "WRITE_SIZE")) for k in kernels)
    f_c = statistics.median(counter_per_dispatch(calib_fetch_dir, fk, "FETCH_SIZE"))
    w_c = statistics.median(counter_per_dispatch(calib_write_dir, calib_kernel, "WRITE_SIZE"))
    f_scale = fb / (f_c * 1024.0)
    w_scale = calib_bytes / (w_c * 1024.0)
    read = f_k * 1024.0 * f_scale
    written = w_k * 1024.0 * w_scale
    return {
        "kernel": kernel,
        "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k,
        "calib_fetch_kernel": fk, "calib_fetch_bytes": fb, "calib_fetch_kib": f_c,
        "calib_write_kernel": calib_kernel, "calib_write_bytes": calib_bytes, "calib_write_kib": w_c,
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "hbm_read_bytes_per_launch": int(read), "hbm_write_bytes_per_launch": int(written),
        "hbm_bytes_per_launch": int(read + written),
    }


def counters(run_dirs: List[str], kernel: str) -> Dict[str, float]:
    """Median per dispatch of every counter collected for kernels matching
    ``kernel`` over one or more ``--pmc`` runs (one pass each)."""
    out: Dict[str, float] = {}
    for d in run_dirs:
        path = _one(os.path.join(d, "**", "*counter_collection.csv"))
        per: Dict[str, List[float]] = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if not per:
            raise ValueError(f"no counters for kernel {kernel!r} in {path}")
        for name, vals in per.items():
            out[name] = statistics.median(vals)
    return out


def _counters_main(a) -> int:
    vals = counters(a.run_dir, a.kernel)
    lines = [f"# {a.title}", "", "Commands (one counter pass each):", ""]
    lines += ["    " + c for c in a.command]
    lines += ["", f"Kernel: `{a.kernel}` (median over its dispatches)", "", "| counter | value |", "|---|---|"]
    for name in sorted(vals):
        v = vals[name]
        lines.append(f"| {name} | {v:.6g} |")
    if a.note:
        lines += ["", a.note]
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)
    return 0


def _stats_main(a) -> int:
    rows = kernel_stats(a.run_dir, a.kernel)
    lines = [f"# {a.title}", "", "Command:", "", "    " + a.command, "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} |")
    if a.note:
        lines += ["", a.note]
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)
    return 0


def _traffic_main(a) -> int:
    rec = traffic(a.fetch, a.write, a.calib_fetch, a.calib_write, a.kernel, a.calib_kernel,
                  a.calib_bytes, a.calib_fetch_kernel, a.calib_fetch_bytes)
    rec["algorithmic_bytes_per_launch"] = a.algorithmic_bytes
    rec["traffic_over_algorithmic"] = round(rec["hbm_bytes_per_launch"] / a.algorithmic_bytes, 4)
    rec["workload"] = a.workload
    rec["source_digest"] = a.source_digest
    rec["commands"] = a.command
    text = json.dumps(rec, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("run_dir")
    s.add_argument("--kernel", action="append", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--out")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "calib_fetch", "calib_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--calib-kernel", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--calib-fetch-kernel", default="")
    t.add_argument("--calib-fetch-bytes", type=int, default=0)
    t.add_argument("--algorithmic-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--source-digest", required=True)
    t.add_argument("--command", action="append", required=True)
    t.add_argument("--out")
    c = sub.add_parser("counters")
    c.add_argument("run_dir", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--title", default="rocprofv3 counters")
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--note", default="")
    c.add_argument("--out")
    a = ap.parse_args(argv)
    return {"stats": _stats_main, "traffic": _traffic_main, "counters": _counters_main}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
