"""Summarise rocprofv3 kernel traces of the skinny GEMM.

    python -m bf16_skinny_gemm_amd.rocprof_summary <out_dir_or_kernel_trace.csv> [--bytes-per-dispatch ...]

Reads the kernel_trace CSV (``rocprofv3 --kernel-trace --output-format csv``)
and prints, per (kernel, grid size, workgroup size), the dispatch count and the
average / min / max duration in microseconds, followed by the per-kernel-name
totals that ``--stats`` reports. Optionally reads the ``--pmc`` counter CSV
(``FETCH_SIZE`` / ``WRITE_SIZE``, in KiB per dispatch) and prints their average
per kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys


def _find(path: str, suffix: str) -> list[str]:
    if os.path.isfile(path):
        return [path]
    return sorted(glob.glob(os.path.join(path, "**", f"*{suffix}"), recursive=True))


def _col(row: dict, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    return None


def kernel_rows(paths):
    for p in paths:
        with open(p, newline="") as f:
            for row in csv.DictReader(f):
                name = _col(row, "Kernel_Name", "KernelName", "Name")
                t0 = _col(row, "Start_Timestamp", "BeginNs", "Start")
                t1 = _col(row, "End_Timestamp", "EndNs", "End")
                if name is None or t0 is None or t1 is None:
                    continue
                grid = _col(row, "Grid_Size_X", "Grid_Size", "grd")
                wg = _col(row, "Workgroup_Size_X", "Workgroup_Size", "wgr")
                yield name, int(grid or 0), int(wg or 0), (int(t1) - int(t0)) / 1000.0


def summarise(trace_paths, filt=None):
    groups = {}
    by_name = {}
    for name, grid, wg, us in kernel_rows(trace_paths):
        if filt and filt not in name:
            continue
        groups.setdefault((name, grid, wg), []).append(us)
        by_name.setdefault(name, []).append(us)
    # p10 / median / p90 over the dispatches: the spread across weight copies (each
    # dispatch of a cell reads a different copy)
    lines = ["dispatches  avg_us   min_us   p10_us   med_us   p90_us   max_us  grid(threads) wg  kernel"]
    for (name, grid, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        q = sorted(v)
        pick = lambda f: q[min(len(q) - 1, int(f * len(q)))]
        lines.append(f"{len(v):10d} {statistics.mean(v):8.3f} {q[0]:8.3f} {pick(0.1):8.3f} "
                     f"{statistics.median(q):8.3f} {pick(0.9):8.3f} {q[-1]:8.3f} "
                     f"{grid:13d} {wg:4d}  {name}")
    lines.append("")
    lines.append("per kernel name (as --stats aggregates):")
    lines.append("dispatches  avg_us   total_us  kernel")
    for name, v in sorted(by_name.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(v):10d} {statistics.mean(v):8.3f} {sum(v):10.1f}  {name}")
    return "\n".join(lines)


def counters(paths, filt=None):
    acc = {}
    for p in paths:
        with open(p, newline="") as f:
            for row in csv.DictReader(f):
                name = _col(row, "Kernel_Name", "KernelName")
                cname = _col(row, "Counter_Name")
                val = _col(row, "Counter_Value")
                if name is None or cname is None or val is None:
                    continue
                if filt and filt not in name:
                    continue
                acc.setdefault((name, cname), []).append(float(val))
    lines = ["counter        dispatches   avg_per_dispatch  kernel"]
    for (name, cname), v in sorted(acc.items()):
        lines.append(f"{cname:14s} {len(v):10d} {statistics.mean(v):18.1f}  {name}")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("path", help="rocprofv3 output directory or a kernel_trace.csv")
    ap.add_argument("--filter", help="only kernels whose name contains this text")
    args = ap.parse_args()
    traces = _find(args.path, "kernel_trace.csv")
    if traces:
        print(summarise(traces, args.filter))
    pmc = _find(args.path, "counter_collection.csv")
    if pmc:
        print()
        print(counters(pmc, args.filter))
    if not traces and not pmc:
        print(f"no rocprofv3 CSV output under {args.path}", file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
