#!/usr/bin/env python3
"""Benchmark of the BF16 skinny GEMM on one MI355X.

One step = one hipGraph replay that runs every (shape, M) cell of the workload,
each over rotated copies of its weight adding up to at least 1 GiB, so that
every call streams its weight from HBM rather than from the 256 MB Infinity
Cache (the cold-cache protocol of vLLM PR #65306, SM90 skinny GEMM plans,
section Validation: graph-captured chains over weight copies of 1 GiB or
more). Inputs are synthetic and seeded (x ~ N(0,1), W ~ N(0,1/K)).

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload kda|single|mla|lm_head|chain]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "cold-cache µs/call and achieved HBM GB/s (% of peak) at M=1/2/4 per (N,K)"
PEAK_HBM_GBPS = 8000.0  # MI355X published HBM3E bandwidth
ROTATE_BYTES = 1 << 30  # >= 1 GiB of weight copies per cell (4x the 256 MB Infinity Cache)

# (name, [(N, K, M), ...]) -- the shapes of the decode projections
WORKLOADS = {
    "kda": ("KDA in_proj (12576,4096) + o_proj (4096,4096) at M=1,2,4, cold cache",
            [(12576, 4096, m) for m in (1, 2, 4)] + [(4096, 4096, m) for m in (1, 2, 4)]),
    "single": ("single skinny GEMM (4096,1024) at M=1, cold cache", [(4096, 1024, 1)]),
    "mla": ("MLA/shared-expert (2048,4096) (4096,1024) (8192,1536) (4096,8192) at M=1,2,4 "
            "+ paired 2x(4096,128), cold cache",
            [(n, k, m) for (n, k) in ((2048, 4096), (4096, 1024), (8192, 1536), (4096, 8192))
             for m in (1, 2, 4)] + [("pair", 4096, 128, m) for m in (1, 2, 4)]),
    "lm_head": ("LM head (77440,4096) at M=1,2,4, cold cache", [(77440, 4096, m) for m in (1, 2, 4)]),
    "kda_m5_8": ("KDA in_proj (12576,4096) + o_proj (4096,4096) at M=5..8, cold cache "
                 "(beyond the decode range the cited plans cover)",
                 [(n, 4096, m) for n in (12576, 4096) for m in (5, 6, 7, 8)]),
}
CHAIN = [(12576, 4096, 34), (4096, 4096, 34), (2048, 4096, 53), (4096, 1024, 42),
         (8192, 1536, 11), (4096, 8192, 11), (77440, 4096, 1)]


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="kda", choices=sorted(list(WORKLOADS) + ["chain"]))
    ap.add_argument("--chain-m", type=int, default=1, help="M of the decode-chain workload")
    ap.add_argument("--trials", type=int, default=5, help="per-cell timing trials")
    ap.add_argument("--replays", type=int, default=20, help="graph replays per per-cell trial")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-oracle sample budget")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch.nn.functional.linear (the vendor BLAS path) on every "
                         "cell under the same graph protocol (informational)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of 256 MiB (PMC counter calibration)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the read-stream ceiling: the read-only probe kernel at "
                         "64 MiB, 256 MiB and 1 GiB per read (rotated over >= 1 GiB), both cache "
                         "hints, several grids; a line fit gives rate and fixed cost per launch")
    return ap.parse_args()


KERNEL_SOURCES = tuple(f"bf16_skinny_gemm_amd/csrc/{f}" for f in (
    "kernels.hpp", "variants.hpp", "skinny_gemm.hip", "variants_fixed_small.hip",
    "variants_fixed_k4096.hip", "variants_fixed_k8192.hip", "variants_other.hip",
    "plans_gfx950.inc"))


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed (string literals
    in these files hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    """Digest of the kernel sources, variant tables and plan table, comments and
    whitespace aside: PMC records taken on other code no longer describe the
    kernels that run."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from profiles/traffic_<workload>.txt, scaled
    by the plain-copy calibration, or None if absent or taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    try:
        if rec.get("source_digest") != source_digest() or rec.get("kernel") != kernel:
            return None
        fetch = float(rec["fetch_kib_per_dispatch"]) * 1024 * float(rec["copy_fetch_factor"])
        write = float(rec["write_kib_per_dispatch"]) * 1024 * float(rec["copy_write_factor"])
    except (KeyError, ValueError):
        return None
    return round(fetch + write)


def copy_calibration() -> int:
    """Plain device-to-device copies of a known size, for scaling FETCH_SIZE and
    WRITE_SIZE: each copy reads and writes exactly 256 MiB."""
    import torch

    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 4}), flush=True)
    return 0


def fit_line(xs, ys):
    """Least-squares y = a + b x; returns (a, b)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    return my - b * mx, b


def read_ceiling(args) -> int:
    """HBM read rate of a kernel that only reads (libskinny_stream_probe.so), the
    practical ceiling beside which the GEMV's weight stream is judged. Reads of
    64 MiB, 256 MiB and 1 GiB, each size rotated over >= 1 GiB of views into one
    2 GiB buffer (past the 256 MB Infinity Cache), one graph of reads per (size,
    cache hint, grid), timed like the cells. Time against bytes is fitted with a
    line: the slope is the streaming rate, the intercept the fixed cost of a
    launch (start-up, ramp and drain)."""
    import torch

    from bf16_skinny_gemm_amd import probe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pool = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    pool.fill_(1)
    sizes = (64 << 20, 256 << 20, 1 << 30)
    rows, fits = [], []
    chunk = 32 << 10  # the probe's chunk: grid 0 below means one block per chunk
    for nt in (True, False):
        for grid_mode in (1024, 2048, 4096, 0):
            per_size = []
            for size in sizes:
                grid = grid_mode or min(65536, size // chunk)
                sink = torch.empty(probe.sink_words(grid), dtype=torch.int32, device=dev)
                views = [pool[i * size:(i + 1) * size] for i in range(max(2, (1 << 30) // size))]

                def run(views=views, sink=sink, nt=nt, grid=grid):
                    for v in views:
                        probe.read(v, sink, nontemporal=nt, grid_blocks=grid)

                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    run()
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s):
                        run()
                torch.cuda.current_stream().wait_stream(s)
                g.replay()
                torch.cuda.synchronize()
                per = []
                for _ in range(args.trials):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(args.replays):
                        g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    per.append(e0.elapsed_time(e1) * 1e3 / (args.replays * len(views)))
                us = statistics.median(per)
                per_size.append(us)
                rows.append({"nontemporal": int(nt), "grid_blocks": grid, "bytes": size,
                             "us_per_read": round(us, 2), "gbps": round(size / (us * 1e-6) / 1e9, 1)})
                log(f"read probe nt={int(nt)} grid={grid} {size >> 20} MiB: {us:.2f} us, "
                    f"{rows[-1]['gbps']} GB/s")
                del g
            a, b = fit_line(list(sizes), per_size)
            fits.append({"nontemporal": int(nt), "grid": grid_mode or "one block per chunk",
                         "stream_gbps": round(1e-3 / b, 1), "fixed_us": round(a, 2)})
            log(f"fit nt={int(nt)} grid={fits[-1]['grid']}: {fits[-1]['stream_gbps']} GB/s + "
                f"{a:.2f} us per launch")
    best = max(fits, key=lambda f: f["stream_gbps"])
    print(json.dumps({"read_ceiling_gbps": best["stream_gbps"], "best_fit": best, "fits": fits,
                      "runs": rows}), flush=True)
    return 0


def bytes_per_call(cell) -> int:
    if cell[0] == "pair":
        _, N, K, M = cell
        return 4 * N * K + 2 * M * K + 4 * M * N
    N, K, M = cell
    return 2 * N * K + 2 * M * K + 2 * M * N


def weight_bytes(cell) -> int:
    """The weight alone, the rate vLLM PR #65306 (section Validation) quotes."""
    if cell[0] == "pair":
        return 4 * cell[1] * cell[2]
    return 2 * cell[0] * cell[1]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cell_name(cell) -> str:
    if cell[0] == "pair":
        return f"pair2x({cell[1]},{cell[2]})M{cell[3]}"
    return f"({cell[0]},{cell[1]})M{cell[2]}"


def kernel_name(p, M) -> str:
    """The kernel instance a plan launches, spelled as rocprofv3 prints it."""
    nt = "true" if p.nontemporal else "false"
    if p.kind == 1:
        xl = p.x_in_lds
        return (f"void skg::fixed_k_kernel<{M}, {p.lanes_per_row}, {p.chunks}, {p.rows_per_wave}, "
                f"{p.k_split}, {xl}, {nt}, {p.prefetch}>(skg::Args)")
    if p.kind == 2:
        return f"void skg::loop_k_kernel<{M}, {p.chunks}, {p.rows_per_wave}, {nt}>(skg::Args, int)"
    if p.kind == 4:
        pf = "true" if p.prefetch else "false"
        return (f"void skg::mfma_kernel<{M}, {p.chunks}, {p.rows_per_wave}, {p.k_split}, {nt}, "
                f"{pf}>(skg::Args)")
    return f"void skg::scalar_kernel<{M}>(skg::Args)"


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. "
              "The GEMV shards by output rows with no exchange, so N GPUs each run one "
              "rank's share at its own shape; run with --gpus 1.", file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration()
    if args.read_ceiling:
        return read_ceiling(args)

    import numpy as np
    import torch

    import bf16_skinny_gemm_amd as skg
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    skg.skinny_gemm_init(0)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def to_host(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    # ---------------- inputs ----------------
    calls = []      # (cell, fn) in step order
    cells = []      # per cell: dict with buffers
    if args.workload == "chain":
        M = args.chain_m
        desc = f"decode-step projection chain, 186 distinct weights, M={M}"
        gen = torch.Generator(device=dev)
        xs = {}
        tid = 0
        for (N, K, count) in CHAIN:
            if K not in xs:
                xs[K] = to_dev(synth.activations(M, K, seed=0, shape_id=K, tensor_id=0))
            ws = []
            for _ in range(count):
                gen.manual_seed(1000 + tid)
                tid += 1
                w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
                w.copy_(torch.randn((N, K), generator=gen, device=dev) * (1.0 / math.sqrt(K)))
                ws.append(w)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            cells.append({"cell": (N, K, M), "x": xs[K], "ws": ws, "y": y, "calls": count})
        log(f"chain weights resident: {sum(c['ws'][0].numel() * 2 * len(c['ws']) for c in cells) / 1e9:.2f} GB")
    else:
        desc, cell_list = WORKLOADS[args.workload]
        for i, cell in enumerate(cell_list):
            if cell[0] == "pair":
                _, N, K, M = cell
                w0 = synth.weights(N, K, seed=0, shape_id=N * 7 + K, tensor_id=1)
                w1 = synth.weights(N, K, seed=0, shape_id=N * 7 + K, tensor_id=2)
                copies = max(1, math.ceil(ROTATE_BYTES / (4 * N * K)))
                W0d, W1d = to_dev(w0), to_dev(w1)
                ws = [(W0d, W1d)] + [(W0d.clone(), W1d.clone()) for _ in range(copies - 1)]
                host_w = (w0, w1)
                y = (torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                     torch.empty((M, N), dtype=torch.bfloat16, device=dev))
            else:
                N, K, M = cell
                wb = synth.weights(N, K, seed=0, shape_id=N * 7 + K, tensor_id=1)
                copies = max(1, math.ceil(ROTATE_BYTES / (2 * N * K)))
                Wd = to_dev(wb)
                ws = [Wd] + [Wd.clone() for _ in range(copies - 1)]
                host_w = wb
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            xb = synth.activations(M, K, seed=0, shape_id=N * 7 + K, tensor_id=0)
            cells.append({"cell": cell, "x": to_dev(xb), "xb": xb, "ws": ws, "y": y,
                          "calls": len(ws), "host_w": host_w})
            log(f"cell {cell_name(cell)}: {len(ws)} weight copies")
    torch.cuda.synchronize()

    def run_cell(c):
        cell = c["cell"]
        if cell[0] == "pair":
            for (w0, w1) in c["ws"]:
                skg.gemm_pair(c["x"], w0, w1, out0=c["y"][0], out1=c["y"][1])
        else:
            for w in c["ws"]:
                skg.gemm(c["x"], w, out=c["y"])

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()  # eager warm-up on the capture stream
            with torch.cuda.graph(g, stream=s):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        return g

    def step_fn():
        for c in cells:
            run_cell(c)

    def time_vendor(c):
        # torch.nn.functional.linear on the same inputs and weight copies, same protocol
        lin = torch.nn.functional.linear

        def run():
            if c["cell"][0] == "pair":
                for (w0, w1) in c["ws"]:
                    lin(c["x"], w0)
                    lin(c["x"], w1)
            else:
                for w in c["ws"]:
                    lin(c["x"], w)

        gv = capture(run)
        gv.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(args.trials):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.replays):
                gv.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / (args.replays * c["calls"]))
        del gv
        return statistics.median(per)

    step_bytes = sum(bytes_per_call(c["cell"]) * c["calls"] for c in cells)
    step_calls = sum(c["calls"] for c in cells)
    log(f"capturing step: {step_calls} launches, {step_bytes / 1e9:.3f} GB per step")
    g_step = capture(step_fn)

    # ---------------- timed steps ----------------
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        g_step.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step: {ms_per_step:.4f} ms, {value:.1f} GB/s (wall {wall:.3f} s for {args.steps} steps)")

    # ---------------- per-cell timing (events on the launch stream) ----------------
    cell_rows = []
    for c in cells:
        g = capture(lambda c=c: run_cell(c))
        g.replay()
        torch.cuda.synchronize()
        per_call = []
        for _ in range(args.trials):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            per_call.append(e0.elapsed_time(e1) * 1e3 / (args.replays * c["calls"]))
        us = statistics.median(per_call)
        b = bytes_per_call(c["cell"])
        gbps = b / (us * 1e-6) / 1e9
        row = {"cell": cell_name(c["cell"]), "us_per_call": round(us, 3),
               "us_min": round(min(per_call), 3), "us_max": round(max(per_call), 3),
               "gbps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
               "weight_gbps": round(weight_bytes(c["cell"]) / (us * 1e-6) / 1e9, 1),
               "bytes_per_call": b, "calls_per_replay": c["calls"]}
        if c["cell"][0] == "pair":
            _, N, K, M = c["cell"]
        else:
            N, K, M = c["cell"]
        p, tuned = skg.skinny_gemm_get_plan(N, K, M)
        row["plan"] = p.as_dict()
        row["tuned_plan"] = tuned
        row["kernel"] = kernel_name(p, M)
        cell_rows.append(row)
        log(f"cell {row['cell']}: {us:.3f} us/call, {gbps:.1f} GB/s ({100 * gbps / PEAK_HBM_GBPS:.1f}% of 8 TB/s)")
        del g
        if args.vendor:
            vus = time_vendor(c)
            row["vendor_us_per_call"] = round(vus, 3)
            row["speedup_vs_vendor"] = round(vus / us, 3)
            log(f"cell {row['cell']}: F.linear {vus:.3f} us/call ({vus / us:.2f}x the skinny GEMM's time)")

    # The dominant kernel: the compiled kernel instance that takes the largest share
    # of the step. Cells that launch the same instance are pooled, so the average
    # launch duration here is the one rocprofv3 --stats reports for that kernel name.
    pooled = {}
    for c, row in zip(cells, cell_rows):
        key = row.get("kernel", row["cell"])
        p = pooled.setdefault(key, {"us": 0.0, "launches": 0, "bytes": 0, "cells": []})
        p["us"] += row["us_per_call"] * c["calls"]
        p["launches"] += c["calls"]
        p["bytes"] += row["bytes_per_call"] * c["calls"]
        p["cells"].append(row["cell"])
    dom_name, dom = max(pooled.items(), key=lambda kv: kv[1]["us"])
    avg_us = dom["us"] / dom["launches"]
    bytes_per_launch = dom["bytes"] / dom["launches"]
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom_name, "cells": dom["cells"],
                "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": recorded_traffic(args.workload, dom_name),
                "avg_launch_us": round(avg_us, 3), "launches_per_step": dom["launches"],
                "algorithmic_bytes_per_launch": round(bytes_per_launch),
                "share_of_step": round(dom["us"] / sum(p["us"] for p in pooled.values()), 4)}

    # ---------------- parity spot check of the timed buffers ----------------
    parity = None
    if not args.no_parity and args.workload != "chain":
        import oracle

        ok = True
        worst = 0.0
        for c in cells:
            cell = c["cell"]
            g = np.random.default_rng(0)
            if cell[0] == "pair":
                N = cell[1]
                rows = np.unique(g.integers(0, N, 256)).astype(np.int64)
                for yt, wb in zip(c["y"], c["host_w"]):
                    yr, ref, mag = oracle.gemm_rows(c["xb"], wb, rows)
                    r = oracle.acceptance(to_host(yt)[:, rows], yr, ref, mag, check_cosine=False)
                    ok &= r["pass"]
                    worst = max(worst, r["max_s1_ratio"])
            else:
                N = cell[0]
                rows = np.unique(np.concatenate([np.arange(min(N, 64)), np.arange(N - 64, N),
                                                 g.integers(0, N, 256)])).astype(np.int64)
                yr, ref, mag = oracle.gemm_rows(c["xb"], c["host_w"], rows)
                r = oracle.acceptance(to_host(c["y"])[:, rows], yr, ref, mag, check_cosine=False)
                ok &= r["pass"]
                worst = max(worst, r["max_s1_ratio"])
        parity = {"pass": bool(ok), "max_s1_ratio": round(worst, 4), "sampled": True}
        log(f"parity spot check: {parity}")

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu and args.workload != "chain":
        import oracle

        nt = oracle.default_threads()
        done_bytes = 0
        t_cpu = 0.0
        passes = 0
        while t_cpu < args.cpu_seconds and passes < 100000:
            for c in cells:
                cell = c["cell"]
                t1 = time.perf_counter()
                if cell[0] == "pair":
                    oracle.gemm_pair(c["xb"], c["host_w"][0], c["host_w"][1], nthreads=nt)
                else:
                    oracle.gemm(c["xb"], c["host_w"], nthreads=nt)
                t_cpu += time.perf_counter() - t1
                done_bytes += bytes_per_call(cell)
            passes += 1
        cpu = {"value": round(done_bytes / t_cpu / 1e9, 3), "unit": "GB/s", "cores": nt,
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"{passes} pass(es) of one call per cell of the workload "
                         f"({len(cells)} cells), fp64 C oracle, {t_cpu:.1f} s"}
        log(f"cpu oracle: {cpu}")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "launches_per_step": step_calls,
                   "bytes_per_step": step_bytes, "rotation_bytes_min": ROTATE_BYTES,
                   "accumulate": "fp32", "device": props.name,
                   "source_digest": source_digest()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cells": cell_rows,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
