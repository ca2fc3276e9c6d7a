"""Summarise rocprofv3 output and benchmark lines of the skinny GEMM.

    python -m bf16_skinny_gemm_amd.rocprof_summary <out_dir_or_kernel_trace.csv> [--filter TEXT]
    python -m bf16_skinny_gemm_amd.rocprof_summary --bench-json BENCH.json
    python -m bf16_skinny_gemm_amd.rocprof_summary --traffic FETCH_DIR WRITE_DIR \
        --copy COPY_FETCH_DIR COPY_WRITE_DIR --kernel NAME --digest HEX

Kernel traces (``rocprofv3 --kernel-trace --output-format csv``): per (kernel,
grid size, workgroup size) the dispatch count and the average / min / p10 /
median / p90 / max duration in microseconds, then the per-kernel-name totals
that ``--stats`` reports; ``--pmc`` counter CSVs (``FETCH_SIZE`` /
``WRITE_SIZE``, KiB per dispatch): their average per kernel.

``--bench-json`` renders the tables of one ``bench.py`` JSON line: the chains
(per shape: event-timed and kernel-trace µs per call), the cells (kernel-trace
duration, replay time per call, dependent chain, the read probe of the same
size, CPU oracle, parity), the read probe per size and the empty-kernel floor.

``--counter-table DIR [DIR ...]`` averages every counter of every ``--pmc`` pass
given (one directory per pass, all over the same command) per (kernel, grid,
workgroup) and prints the derived figures: loaded vector-memory latency, scalar
(kernel-argument) load latency, mean waves per CU, translation-miss rate, L1→L2
and L2→DRAM request latencies.

``--traffic`` writes the HBM-traffic record ``bench.py`` reads for its roofline:
the average FETCH_SIZE and WRITE_SIZE per dispatch of one kernel (all of its
dispatches, in the proportions the profiled command launched them), and the
factors that turn each counter into bytes, from a plain device copy of
256 MiB profiled the same way (``bench.py --copy-calibration``).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
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


def _counter_avg(paths, counter, name_filter):
    vals = []
    for p in paths:
        with open(p, newline="") as f:
            for row in csv.DictReader(f):
                if _col(row, "Counter_Name") != counter:
                    continue
                name = _col(row, "Kernel_Name", "KernelName") or ""
                if name_filter(name):
                    vals.append(float(_col(row, "Counter_Value")))
    return (statistics.mean(vals) if vals else None), len(vals)


COPY_BYTES = 256 << 20  # bench.py --copy-calibration copies this many bytes


def traffic_record(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kernel, digest):
    """The traffic record: KiB per dispatch of `kernel` and the copy factors."""
    f, nf = _counter_avg(_find(fetch_dir, "counter_collection.csv"), "FETCH_SIZE", lambda n: n == kernel)
    w, nw = _counter_avg(_find(write_dir, "counter_collection.csv"), "WRITE_SIZE", lambda n: n == kernel)
    is_copy = lambda n: "copyBuffer" in n
    cf, _ = _counter_avg(_find(copy_fetch_dir, "counter_collection.csv"), "FETCH_SIZE", is_copy)
    cw, _ = _counter_avg(_find(copy_write_dir, "counter_collection.csv"), "WRITE_SIZE", is_copy)
    if None in (f, w, cf, cw):
        raise SystemExit("missing counters: FETCH_SIZE/WRITE_SIZE of the kernel or of the copy")
    kib = COPY_BYTES / 1024.0
    lines = [f"source_digest: {digest}", f"kernel: {kernel}",
             f"fetch_kib_per_dispatch: {f:.3f}", f"write_kib_per_dispatch: {w:.3f}",
             f"dispatches: {nf} (FETCH_SIZE run), {nw} (WRITE_SIZE run)",
             f"copy_fetch_factor: {kib / cf:.5f}", f"copy_write_factor: {kib / cw:.5f}",
             f"hbm_bytes_per_dispatch: {f * 1024 * kib / cf + w * 1024 * kib / cw:.0f}"]
    return "\n".join(lines)


def counter_table(dirs, filt="skg::"):
    """Per (kernel, grid, workgroup): the mean of each counter over its dispatches,
    pooled over the passes in `dirs`, and the figures derived from them."""
    acc = {}
    for d in dirs:
        for p in _find(d, "counter_collection.csv"):
            with open(p, newline="") as f:
                for row in csv.DictReader(f):
                    name = _col(row, "Kernel_Name") or ""
                    if filt and filt not in name:
                        continue
                    key = (name, int(_col(row, "Grid_Size") or 0), int(_col(row, "Workgroup_Size") or 0))
                    acc.setdefault(key, {}).setdefault(_col(row, "Counter_Name"), []).append(
                        float(_col(row, "Counter_Value")))
    out = []
    for (name, grid, wg), c in sorted(acc.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        m = {k: statistics.mean(v) for k, v in c.items()}
        g = lambda k: m.get(k, float("nan"))
        miss, hit = g("TCP_UTCL1_TRANSLATION_MISS_sum"), g("TCP_UTCL1_TRANSLATION_HIT_sum")
        out.append(f"{name.replace('void skg::', '').replace('(skg::Args)', '')}  blocks={grid // max(1, wg)} x {wg}")
        out.append(f"    waves {g('SQ_WAVES'):.0f}, mean waves per CU {g('MeanOccupancyPerCU'):.1f}; "
                   f"vector-memory latency {g('VmemLatency'):.0f} cycles, scalar-load latency "
                   f"{g('SmemLatency'):.0f} cycles ({g('SQ_INSTS_SMEM') / max(1.0, g('SQ_WAVES')):.1f} per wave), "
                   f"LDS latency {g('LdsLatency'):.0f} cycles, LDS bank-conflict cycles {g('SQ_LDS_BANK_CONFLICT'):.0f}")
        out.append(f"    UTCL1 translations: {miss:.0f} misses / {hit:.0f} hits "
                   f"({100 * miss / max(1.0, miss + hit):.2f}% miss); L1->L2 read latency "
                   f"{g('TCP_TCC_READ_REQ_LATENCY_sum') / max(1.0, g('TCP_TCC_READ_REQ_sum')):.0f} cycles over "
                   f"{g('TCP_TCC_READ_REQ_sum'):.0f} requests; L2->DRAM read latency "
                   f"{g('TCC_EA0_RDREQ_LEVEL_sum') / max(1.0, g('TCC_EA0_RDREQ_sum')):.0f} cycles over "
                   f"{g('TCC_EA0_RDREQ_sum'):.0f} requests; L2 hits {g('TCC_HIT_sum'):.0f}, misses {g('TCC_MISS_sum'):.0f}")
        out.append(f"    instructions per wave: vmem reads {g('SQ_INSTS_VMEM_RD') / max(1.0, g('SQ_WAVES')):.1f}, "
                   f"valu {g('SQ_INSTS_VALU') / max(1.0, g('SQ_WAVES')):.0f}, salu {g('SQ_INSTS_SALU') / max(1.0, g('SQ_WAVES')):.0f}; "
                   f"TA busy {g('TA_TA_BUSY_sum'):.0f}, TD busy {g('TD_TD_BUSY_sum'):.0f}, "
                   f"GRBM_GUI_ACTIVE {g('GRBM_GUI_ACTIVE'):.0f}")
    return "\n".join(out)


def _fmt(v, nd=3):
    return "n/a" if v is None else (f"{v:.{nd}f}" if isinstance(v, float) else str(v))


def bench_tables(d):
    """Markdown tables of one bench.py JSON line."""
    out = []
    for c in d.get("chains", []):
        out.append(f"### Decode-step chain, M = {c['M']}: {c['ms_per_step'] * 1e3:.1f} µs per step of "
                   f"{c['calls']} calls, {c['gbps']} GB/s ({100 * c['frac_of_peak']:.1f}% of 8 TB/s)")
        if "parity" in c:
            p = c["parity"]
            out.append(f"parity: pass={p['pass']}, {p['outputs_checked']} outputs, {p['elements']} "
                       f"elements, max G1 ratio {p['max_g1_ratio']}, max S1 ratio {p['max_s1_ratio']}, "
                       f"min row cosine {p['min_row_cosine']:.9f}")
        out.append("")
        out.append("| shape | calls | kernel | event µs/call | % of 8 TB/s | rocprof avg µs | rocprof % |")
        out.append("|---|---|---|---|---|---|---|")
        for g in c["groups"]:
            rp = g.get("rocprof", {})
            out.append(f"| {g['shape']} | {g['calls']} | `{g['kernel'].replace('void skg::', '')}` | "
                       f"{_fmt(g.get('event_us_per_call'))} | {_fmt(100 * g['event_frac'], 1) if 'event_frac' in g else 'n/a'} | "
                       f"{_fmt(rp.get('avg_us'))} | {_fmt(100 * g['kernel_frac'], 1) if 'kernel_frac' in g else 'n/a'} |")
        out.append("")
    if d.get("cells"):
        out.append("### Cells (cold cache, >= 1 GiB of rotated copies)")
        out.append("")
        vendor = any("vendor_us_per_call" in c for c in d["cells"])
        out.append("| cell | rocprof avg µs (med) | % of 8 TB/s | replay µs/call | % | dependent µs/call | "
                   "read probe µs (replay) | replay ÷ probe | CPU oracle µs | parity |"
                   + (" F.linear µs/call | F.linear ÷ skinny |" if vendor else ""))
        out.append("|---|---|---|---|---|---|---|---|---|---|" + ("---|---|" if vendor else ""))
        for c in d["cells"]:
            rp = c.get("rocprof", {})
            kern = f"{_fmt(rp.get('avg_us'))} ({_fmt(rp.get('med_us'))})" if rp else "n/a"
            ratio = (c["replay_us_per_call"] / c["read_probe_replay_us"]) if c.get("read_probe_replay_us") else None
            out.append(f"| {c['cell']} | {kern} | {_fmt(100 * c['kernel_frac'], 1) if 'kernel_frac' in c else 'n/a'} | "
                       f"{c['replay_us_per_call']:.3f} | {100 * c['replay_frac']:.1f} | "
                       f"{_fmt(c.get('dependent_us_per_call'))} | {_fmt(c.get('read_probe_replay_us'))} | "
                       f"{_fmt(ratio)} | {_fmt(c.get('cpu_oracle_us'), 1)} | "
                       f"{c.get('parity', {}).get('pass', 'n/a')} |"
                       + (f" {_fmt(c.get('vendor_us_per_call'))} | {_fmt(c.get('speedup_vs_vendor'))} |"
                          if vendor else ""))
        out.append("")
    if d.get("read_probe"):
        out.append("### Read-only probe (one block per tile, each size over >= 1 GiB of buffers)")
        out.append("")
        out.append("| bytes | best shape (loads x threads) | replay µs | GB/s | rocprof best µs | all shapes: replay µs |")
        out.append("|---|---|---|---|---|---|")
        for r in d["read_probe"]:
            b = r["best_replay"]
            allr = ", ".join(f"{a['loads']}x{a['threads']}: {a['replay_us']}" for a in r["all"])
            out.append(f"| {r['bytes']} | {b['loads']}x{b['threads']} | {b['replay_us']} | {r['replay_gbps']} | "
                       f"{_fmt(r.get('best_kernel', {}).get('kernel_us'))} | {allr} |")
        out.append("")
    if d.get("empty_kernel"):
        out.append("### Empty kernel (256 threads per block), per launch")
        out.append("")
        out.append("| blocks | replay µs per launch | rocprof avg µs |")
        out.append("|---|---|---|")
        for e in d["empty_kernel"]:
            out.append(f"| {e['grid']} | {e['replay_us_per_launch']} | {_fmt(e.get('kernel_us'))} |")
        out.append("")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("path", nargs="?", help="rocprofv3 output directory or a kernel_trace.csv")
    ap.add_argument("--filter", help="only kernels whose name contains this text")
    ap.add_argument("--bench-json", help="render the tables of a bench.py JSON line")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--copy", nargs=2, metavar=("COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--counter-table", nargs="+", metavar="DIR")
    ap.add_argument("--kernel", help="kernel name for --traffic")
    ap.add_argument("--digest", help="source digest for --traffic (bench.source_digest())")
    args = ap.parse_args()
    if args.bench_json:
        with open(args.bench_json) as f:
            line = [l for l in f if l.strip().startswith("{")][-1]
        print(bench_tables(json.loads(line)))
        return 0
    if args.counter_table:
        print(counter_table(args.counter_table, args.filter or "skg::"))
        return 0
    if args.traffic:
        if not (args.copy and args.kernel and args.digest):
            ap.error("--traffic needs --copy, --kernel and --digest")
        print(traffic_record(*args.traffic, *args.copy, args.kernel, args.digest))
        return 0
    if not args.path:
        ap.error("give a rocprofv3 output path, --bench-json or --traffic")
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
