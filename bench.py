#!/usr/bin/env python3
"""Benchmark of the BF16 skinny GEMM on one MI355X.

Default workload: the decode-step projection chain, 186 calls with distinct
weights in the order (12576,4096) x34, (4096,4096) x34, (2048,4096) x53,
(4096,1024) x42, (8192,1536) x11, (4096,8192) x11, (77440,4096) x1 (7.53 GB of
weights, the per-step call counts of vLLM PR #62949, SM121 skinny GEMM plans,
section Validation), captured in one hipGraph. One step is one replay of the
chain at M = 1; `value` is its algorithmic bytes per second. The same chain at
M = 4 is timed beside it, and every single-shape cell of the other workloads
((4096,1024) at M = 1; the KDA in_proj/o_proj, the MLA/shared-expert shapes,
the paired (4096,128) weights and the LM head at M = 1, 2, 4) is timed on its
own over rotated weight copies of at least 1 GiB, so that each call streams its
weight from HBM rather than from the 256 MB Infinity Cache (the cold-cache
protocol of vLLM PR #65306, SM90 skinny GEMM plans, section Validation:
graph-captured chains over >= 1 GiB of weight copies, 11 trials x 300 replays).

Per cell it reports the kernel duration from a rocprofv3 kernel trace (a child
pass of this script run under `rocprofv3 --kernel-trace`, skipped when the
script already runs under a profiler), the event-timed replay time per call,
the same calls as a dependent chain (x of call i+1 = the first M*K outputs of
call i) where N >= K, the read-only probe's time for the same number of bytes,
the CPU oracle's time and parity of the timed outputs against the oracle. Inputs
are synthetic and seeded (x ~ N(0,1), W ~ N(0,1/K)).

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload chain|kda|single|mla|lm_head|kda_m5_8]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import shutil
import statistics
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "cold-cache µs/call and achieved HBM GB/s (% of peak) at M=1/2/4 per (N,K)"
PEAK_HBM_GBPS = 8000.0  # MI355X published HBM3E bandwidth
ROTATE_BYTES = 1 << 30  # >= 1 GiB of weight copies per cell (4x the 256 MB Infinity Cache)

# The decode-step chain: (N, K, calls per step), in call order.
CHAIN = [(12576, 4096, 34), (4096, 4096, 34), (2048, 4096, 53), (4096, 1024, 42),
         (8192, 1536, 11), (4096, 8192, 11), (77440, 4096, 1)]
CHAIN_DESC = ("decode-step projection chain: 186 distinct seeded weights, (12576,4096)x34, "
              "(4096,4096)x34, (2048,4096)x53, (4096,1024)x42, (8192,1536)x11, (4096,8192)x11, "
              "(77440,4096)x1, 7.53 GB, one hipGraph")

# Single-shape cells: shape key -> (token counts, configurations they belong to).
# A shape key is (N, K) or ("pair", N, K) for two same-shape weights on one x.
CELL_SHAPES = [
    ((4096, 1024), (1, 2, 4), "single (4096,1024) M=1; MLA/shared-expert"),
    ((12576, 4096), (1, 2, 4), "KDA in_proj"),
    ((4096, 4096), (1, 2, 4), "KDA o_proj"),
    ((2048, 4096), (1, 2, 4), "MLA/shared-expert"),
    ((8192, 1536), (1, 2, 4), "MLA/shared-expert"),
    ((4096, 8192), (1, 2, 4), "MLA/shared-expert"),
    (("pair", 4096, 128), (1, 2, 4), "paired f_b/g_b"),
    ((77440, 4096), (1, 2, 4), "LM head"),
]

# Workloads that time a set of cells as the step (no chain).
CELL_WORKLOADS = {
    "kda": ("KDA in_proj (12576,4096) + o_proj (4096,4096) at M=1,2,4, cold cache",
            [((12576, 4096), (1, 2, 4)), ((4096, 4096), (1, 2, 4))]),
    "single": ("single skinny GEMM (4096,1024) at M=1, cold cache", [((4096, 1024), (1,))]),
    "mla": ("MLA/shared-expert (2048,4096) (4096,1024) (8192,1536) (4096,8192) at M=1,2,4 "
            "+ paired 2x(4096,128), cold cache",
            [((2048, 4096), (1, 2, 4)), ((4096, 1024), (1, 2, 4)), ((8192, 1536), (1, 2, 4)),
             ((4096, 8192), (1, 2, 4)), (("pair", 4096, 128), (1, 2, 4))]),
    "lm_head": ("LM head (77440,4096) at M=1,2,4, cold cache", [((77440, 4096), (1, 2, 4))]),
    "kda_m5_8": ("KDA in_proj (12576,4096) + o_proj (4096,4096) at M=5..8, cold cache "
                 "(beyond the decode range the cited plans cover)",
                 [((12576, 4096), (5, 6, 7, 8)), ((4096, 4096), (5, 6, 7, 8))]),
}

# The read-only probe's shapes (loads per lane, threads per block) tried at each size.
PROBE_SHAPES = ((4, 256), (8, 256), (2, 256), (4, 512), (16, 256))
# Grid sizes of the empty kernel (256 threads per block) for the per-launch floor.
EMPTY_GRIDS = (1, 256, 1024, 4096, 16384, 65536)
EMPTY_LAUNCHES = 1000

# Kernel-trace pass: replays per unit (the rocprofv3 durations are per dispatch).
TRACE_REPLAYS = {"chain": 10, "cell": 10, "dep": 5, "probe": 3, "empty": 1}


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300, help="timed replays of the step")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="chain", choices=["chain", "cells"] + sorted(CELL_WORKLOADS))
    ap.add_argument("--only", help="cells workload: shapes to run, e.g. 4096x4096,2048x4096 or pair4096x128")
    ap.add_argument("--ms", default="1,2,4", help="cells workload: token counts")
    ap.add_argument("--chain-ms", default="1,4", help="token counts of the chain; the first is `value`")
    ap.add_argument("--trials", type=int, default=11, help="per-cell timing trials")
    ap.add_argument("--replays", type=int, default=300, help="graph replays per per-cell trial")
    ap.add_argument("--no-cells", action="store_true", help="chain only: skip the single-shape cells")
    ap.add_argument("--no-dependent", action="store_true", help="skip the dependent-chain timings")
    ap.add_argument("--no-probe", action="store_true", help="skip the read probe and empty-kernel floor")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-trace", action="store_true",
                    help="skip the rocprofv3 kernel-trace child pass (kernel durations per cell)")
    ap.add_argument("--trace-dir", help="keep the child pass's rocprofv3 output here")
    ap.add_argument("--trace-pass", action="store_true",
                    help="(internal) replay every unit a few times between markers, for a kernel trace")
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch.nn.functional.linear on every cell (informational)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of 256 MiB (PMC counter calibration)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only run the read probe at every weight size and the empty-kernel floor")
    return ap.parse_args(argv)


KERNEL_SOURCES = tuple(f"bf16_skinny_gemm_amd/csrc/{f}" for f in (
    "kernels.hpp", "variants.hpp", "validate.hpp", "skinny_gemm.hip", "variants_fixed_small.hip",
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


def bytes_per_call(cell) -> int:
    """Algorithmic bytes of one call: the weight(s) once, x once, y once."""
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


def chain_bytes(M: int) -> int:
    return sum(bytes_per_call((N, K, M)) * n for (N, K, n) in CHAIN)


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


def shape_cell(shape, M):
    return (*shape, M)


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


def dist(values):
    """avg / median / p10 / p90 / min / max of a list of microsecond figures."""
    q = sorted(values)
    pick = lambda f: q[min(len(q) - 1, int(f * len(q)))]
    return {"avg_us": round(statistics.mean(q), 3), "med_us": round(statistics.median(q), 3),
            "p10_us": round(pick(0.1), 3), "p90_us": round(pick(0.9), 3),
            "min_us": round(q[0], 3), "max_us": round(q[-1], 3), "n": len(q)}


def rate(nbytes, us):
    gbps = nbytes / (us * 1e-6) / 1e9
    return round(gbps, 1), round(gbps / PEAK_HBM_GBPS, 4)


# ---------------------------------------------------------------------------
# units: one captured graph each, grouped by the weights they share
# ---------------------------------------------------------------------------

class Unit:
    """One captured graph: `launches` kernel launches per replay.

    kind: chain (the decode chain at one M), group (a chain's calls of one shape,
    timed for the dominant kernel; not traced), cell (one shape and M over its
    rotated copies), dep (the same calls, each taking the previous output as x),
    probe (read-only probe over one size), empty (empty kernels).
    """

    def __init__(self, name, kind, graph, launches, nbytes, keep=(), **meta):
        self.name, self.kind, self.graph, self.launches, self.nbytes = name, kind, graph, launches, nbytes
        # every tensor the graph reads or writes: a captured graph holds raw device
        # addresses only, so a tensor it uses must stay referenced while it replays
        self.keep = keep
        self.meta = meta


class Ctx:
    def __init__(self, args):
        import numpy as np
        import torch

        import bf16_skinny_gemm_amd as skg

        self.np, self.torch, self.skg = np, torch, skg
        self.args = args
        self.capture_stream = None
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        skg.skinny_gemm_init(0)

    def to_dev(self, bits):
        np, torch = self.np, self.torch
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(self.dev)

    def to_host(self, t):
        np, torch = self.np, self.torch
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def capture(self, fn):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        if self.capture_stream is None:
            self.capture_stream = torch.cuda.Stream()
        s = self.capture_stream
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()  # eager warm-up on the capture stream
            with torch.cuda.graph(g, stream=s):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        return g

    def time_graph(self, g, trials, replays):
        """Microseconds per replay, one figure per trial (HIP events on the stream
        the graph is launched on)."""
        torch = self.torch
        g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(trials):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / replays)
        return per


def chain_ms(args):
    return [int(m) for m in args.chain_ms.split(",") if m.strip()]


def chain_group(ctx, with_groups: bool):
    """The chain's 186 distinct weights (drawn on the GPU) and, per M, a graph of
    all calls; with_groups adds one graph per shape (the chain's calls of that
    shape alone), for the per-kernel time of the dominant kernel."""
    import synth

    torch = ctx.torch
    weights, calls = [], []
    tid = 0
    for (N, K, count) in CHAIN:
        for _ in range(count):
            weights.append(synth.device_weights(N, K, seed=0, tensor_id=1000 + tid, device=ctx.dev))
            calls.append((N, K))
            tid += 1
    torch.cuda.synchronize()
    log(f"chain weights resident: {sum(w.numel() * 2 for w in weights) / 1e9:.2f} GB")
    units, state = [], {"weights": weights, "calls": calls, "runs": {}}
    for M in chain_ms(ctx.args):
        xb = {K: synth.activations(M, K, seed=0, shape_id=K, tensor_id=0) for K in {k for _, k in calls}}
        xs = {K: ctx.to_dev(b) for K, b in xb.items()}
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=ctx.dev) for (N, _) in calls]

        def run(lo=0, hi=len(calls), xs=xs, ys=ys):
            for i in range(lo, hi):
                ctx.skg.gemm(xs[calls[i][1]], weights[i], out=ys[i])

        state["runs"][M] = {"xb": xb, "ys": ys}
        keep = (xs, ys, weights)
        units.append(Unit(f"chain:M{M}", "chain", ctx.capture(run), len(calls), chain_bytes(M), keep, M=M))
        if with_groups:
            lo = 0
            for (N, K, count) in CHAIN:
                g = ctx.capture(lambda lo=lo, hi=lo + count: run(lo, hi))
                units.append(Unit(f"group:({N},{K})M{M}", "group", g, count,
                                  bytes_per_call((N, K, M)) * count, keep, M=M, N=N, K=K, first=lo))
                lo += count
    return units, state


def cell_group(ctx, shape, Ms, dependent: bool):
    """Rotated copies (>= 1 GiB) of one shape's weight(s), shared by its token
    counts: per M one graph over every copy, and where N >= K a dependent chain
    over the same copies (x of call i+1 = the first M*K outputs of call i)."""
    import synth

    torch = ctx.torch
    pair = shape[0] == "pair"
    N, K = (shape[1], shape[2]) if pair else shape
    sid = N * 7 + K
    if pair:
        host_w = (synth.weights(N, K, seed=0, shape_id=sid, tensor_id=1),
                  synth.weights(N, K, seed=0, shape_id=sid, tensor_id=2))
        copies = max(1, math.ceil(ROTATE_BYTES / (4 * N * K)))
        W0, W1 = ctx.to_dev(host_w[0]), ctx.to_dev(host_w[1])
        ws = [(W0, W1)] + [(W0.clone(), W1.clone()) for _ in range(copies - 1)]
    else:
        host_w = synth.weights(N, K, seed=0, shape_id=sid, tensor_id=1)
        copies = max(1, math.ceil(ROTATE_BYTES / (2 * N * K)))
        Wd = ctx.to_dev(host_w)
        ws = [Wd] + [Wd.clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()
    units, state = [], {"host_w": host_w, "runs": {}}
    for M in Ms:
        cell = shape_cell(shape, M)
        xb = synth.activations(M, K, seed=0, shape_id=sid, tensor_id=0)
        x = ctx.to_dev(xb)
        if pair:
            y = (torch.empty((M, N), dtype=torch.bfloat16, device=ctx.dev),
                 torch.empty((M, N), dtype=torch.bfloat16, device=ctx.dev))

            def run(x=x, y=y):
                for (w0, w1) in ws:
                    ctx.skg.gemm_pair(x, w0, w1, out0=y[0], out1=y[1])
        else:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=ctx.dev)

            def run(x=x, y=y):
                for w in ws:
                    ctx.skg.gemm(x, w, out=y)
        state["runs"][M] = {"xb": xb, "y": y, "x": x, "ws": ws}
        units.append(Unit(f"cell:{cell_name(cell)}", "cell", ctx.capture(run), len(ws),
                          bytes_per_call(cell) * len(ws), (x, y, ws), cell=cell, copies=len(ws)))
        if dependent and N >= K:
            # each call its own output; the first M*K of them are the next call's x
            outs = [torch.empty((M, N), dtype=torch.bfloat16, device=ctx.dev) for _ in ws]
            outs1 = [torch.empty((M, N), dtype=torch.bfloat16, device=ctx.dev) for _ in ws] if pair else None
            for o in outs:
                o.normal_()
            xs = [o.view(-1)[:M * K].view(M, K) for o in outs]

            def run_dep(xs=xs, outs=outs, outs1=outs1):
                n = len(ws)
                for i in range(n):
                    xi = xs[(i - 1) % n]
                    if pair:
                        ctx.skg.gemm_pair(xi, ws[i][0], ws[i][1], out0=outs[i], out1=outs1[i])
                    else:
                        ctx.skg.gemm(xi, ws[i], out=outs[i])
            units.append(Unit(f"dep:{cell_name(cell)}", "dep", ctx.capture(run_dep), len(ws),
                              bytes_per_call(cell) * len(ws), (xs, outs, outs1, ws), cell=cell,
                              copies=len(ws)))
    return units, state


def probe_sizes():
    """Distinct weight sizes of the cells (the pair: both weights), with the shapes they serve."""
    sizes = {}
    for shape, _, _ in CELL_SHAPES:
        nb = 4 * shape[1] * shape[2] if shape[0] == "pair" else 2 * shape[0] * shape[1]
        sizes.setdefault(nb, []).append(shape)
    return sizes


def floor_group(ctx):
    """The read-only probe at each weight size (every probe shape), over >= 1 GiB of
    separately allocated buffers per size, as the cells rotate separately
    allocated weight copies; and the empty kernel at each grid."""
    from bf16_skinny_gemm_amd import probe

    torch = ctx.torch
    units = []
    for nb in sorted(probe_sizes()):
        nviews = probe_copies(nb)
        # random bytes, like the weights the cells stream (not a constant pattern)
        views = [torch.randint(0, 256, (nb,), dtype=torch.uint8, device=ctx.dev) for _ in range(nviews)]
        for loads, threads in PROBE_SHAPES:
            words = probe.tiles_sink_words(nb, loads, threads)
            sink = torch.empty(words, dtype=torch.int32, device=ctx.dev)

            def run(views=views, sink=sink, loads=loads, threads=threads):
                for v in views:
                    probe.read_tiles(v, sink, loads=loads, threads=threads, nontemporal=True)
            units.append(Unit(f"probe:{nb}:{loads}x{threads}", "probe", ctx.capture(run), len(views),
                              nb * len(views), (views, sink), size=nb, loads=loads, threads=threads))
        del views
    for grid in EMPTY_GRIDS:
        def run_empty(grid=grid):
            for _ in range(EMPTY_LAUNCHES):
                probe.empty(grid, 256)
        units.append(Unit(f"empty:{grid}", "empty", ctx.capture(run_empty), EMPTY_LAUNCHES, 0, grid=grid))
    return units, {}


def probe_copies(nb):
    """Buffers the probe rotates over at one size: >= 1 GiB, at least two."""
    return max(2, math.ceil(ROTATE_BYTES / nb))


def unit_groups(ctx, cell_shapes, with_chain, with_groups, dependent, with_probe):
    """Yields (group name, units, state) one group at a time, in a fixed order
    that the trace pass and the timing pass share; a group's device memory is
    released when the next one is built."""
    if with_chain:
        units, state = chain_group(ctx, with_groups)
        yield "chain", units, state
        del units, state
    for shape, Ms in cell_shapes:
        units, state = cell_group(ctx, shape, Ms, dependent)
        yield f"shape:{shape}", units, state
        del units, state
    if with_probe:
        units, state = floor_group(ctx)
        yield "floor", units, state


def plan_of(ctx, cell):
    if cell[0] == "pair":
        _, N, K, M = cell
    else:
        N, K, M = cell
    p, tuned = ctx.skg.skinny_gemm_get_plan(N, K, M)
    return p, tuned, kernel_name(p, M)


# ---------------------------------------------------------------------------
# the kernel-trace pass (a child process under rocprofv3)
# ---------------------------------------------------------------------------

MARKER = "zero_kernel"  # the library's K = 0 kernel: launched only as a separator here
TRACED_KERNELS = ("skg::", "read_tiles_kernel", "empty_kernel")


def shape_key(text):
    """'4096x1024' -> (4096, 1024); 'pair4096x128' -> ('pair', 4096, 128)."""
    t = text.strip()
    pair = t.startswith("pair")
    n, k = (int(v) for v in t[4 if pair else 0:].split("x"))
    return ("pair", n, k) if pair else (n, k)


def traced_units(args):
    """Selection flags shared by the parent and the trace child."""
    if args.workload == "chain":
        cells = [] if args.no_cells else [(s, m) for s, m, _ in CELL_SHAPES]
        return cells, True
    if args.workload == "cells":
        ms = tuple(int(m) for m in args.ms.split(","))
        shapes = [shape_key(t) for t in args.only.split(",")] if args.only else [s for s, _, _ in CELL_SHAPES]
        return [(s, ms) for s in shapes], False
    return CELL_WORKLOADS[args.workload][1], False


def trace_pass(args) -> int:
    """Replays every unit TRACE_REPLAYS[kind] times after a marker launch, so that
    a kernel trace can be cut into units: the dispatches between marker k and
    marker k+1 are unit k's."""
    ctx = Ctx(args)
    torch = ctx.torch
    xm = torch.empty((1, 0), dtype=torch.bfloat16, device=ctx.dev)
    wm = torch.empty((1, 0), dtype=torch.bfloat16, device=ctx.dev)
    ym = torch.empty((1, 1), dtype=torch.bfloat16, device=ctx.dev)
    cells, with_chain = traced_units(args)
    n = 0
    for gname, units, _ in unit_groups(ctx, cells, with_chain, False, not args.no_dependent,
                                       not args.no_probe):
        for u in units:
            # a marker on each side: whatever runs between units (the next group's
            # eager warm-ups) falls between a closing and an opening marker
            torch.cuda.synchronize()
            ctx.skg.gemm(xm, wm, out=ym)
            torch.cuda.synchronize()
            for _ in range(TRACE_REPLAYS[u.kind]):
                u.graph.replay()
            torch.cuda.synchronize()
            ctx.skg.gemm(xm, wm, out=ym)
            torch.cuda.synchronize()
            n += 1
        log(f"trace pass: {gname} done ({n} units)")
        del units
    return 0


def under_profiler() -> bool:
    return any(k.startswith("ROCPROF_") for k in os.environ) or "rocprofiler" in os.environ.get("LD_PRELOAD", "")


def read_kernel_trace(paths):
    """(start_ns, end_ns, name) of every dispatch in rocprofv3 kernel_trace CSVs,
    in launch order."""
    rows = []
    for p in paths:
        with open(p, newline="") as f:
            for row in csv.DictReader(f):
                low = {k.lower(): v for k, v in row.items()}
                name = low.get("kernel_name")
                t0, t1 = low.get("start_timestamp"), low.get("end_timestamp")
                if name is None or t0 is None or t1 is None:
                    continue
                did = low.get("dispatch_id")
                rows.append((int(t0), int(did) if did not in (None, "") else 0, int(t1), name))
    rows.sort()
    return [(t0, t1, name) for (t0, _, t1, name) in rows]


def split_trace(rows, expected):
    """Cut a launch-ordered trace at the marker dispatches. Each unit's replays
    sit between an opening and a closing marker, so the stretches between
    markers alternate: unit, gap (other work), unit, gap, ... `expected` lists
    (unit name, dispatches) in the order the units were replayed. Returns
    {unit name: [duration_us of each of its dispatches, in order]}, leaving out a
    unit whose stretch does not hold exactly the dispatches expected."""
    segs, cur = [], None
    for (t0, t1, name) in rows:
        if MARKER in name:
            cur = []
            segs.append(cur)
        elif cur is not None and any(k in name for k in TRACED_KERNELS):
            cur.append((t1 - t0) / 1000.0)
    out = {}
    for (uname, count), seg in zip(expected, segs[0::2]):
        if len(seg) == count:
            out[uname] = seg
    return out


def expected_trace_units(args):
    """(unit name, dispatches) in trace order, without touching a GPU."""
    cells, with_chain = traced_units(args)
    out = []
    if with_chain:
        for M in chain_ms(args):
            out.append((f"chain:M{M}", len(CHAIN_CALLS) * TRACE_REPLAYS["chain"]))
    for shape, Ms in cells:
        pair = shape[0] == "pair"
        N, K = (shape[1], shape[2]) if pair else shape
        copies = max(1, math.ceil(ROTATE_BYTES / ((4 if pair else 2) * N * K)))
        for M in Ms:
            cell = shape_cell(shape, M)
            out.append((f"cell:{cell_name(cell)}", copies * TRACE_REPLAYS["cell"]))
            if not args.no_dependent and N >= K:
                out.append((f"dep:{cell_name(cell)}", copies * TRACE_REPLAYS["dep"]))
    if not args.no_probe:
        for nb in sorted(probe_sizes()):
            for loads, threads in PROBE_SHAPES:
                out.append((f"probe:{nb}:{loads}x{threads}", probe_copies(nb) * TRACE_REPLAYS["probe"]))
        for grid in EMPTY_GRIDS:
            out.append((f"empty:{grid}", EMPTY_LAUNCHES * TRACE_REPLAYS["empty"]))
    return out


CHAIN_CALLS = [(N, K) for (N, K, n) in CHAIN for _ in range(n)]


def run_trace_child(args):
    """Run this script's trace pass under `rocprofv3 --kernel-trace` in a child
    process (before this process touches the GPU) and return the per-unit
    dispatch durations, or None with the reason logged."""
    exe = shutil.which("rocprofv3")
    if exe is None:
        log("kernel trace: rocprofv3 not found, per-cell kernel durations left out")
        return None, "rocprofv3 not found"
    # absolute: the child runs with /tmp as its working directory
    out_dir = os.path.abspath(args.trace_dir) if args.trace_dir else tempfile.mkdtemp(prefix="skinny_trace_",
                                                                                      dir="/tmp")
    os.makedirs(out_dir, exist_ok=True)
    cmd = [exe, "--kernel-trace", "--stats", "--output-format", "csv", "-d", out_dir, "-o", "trace",
           "--", sys.executable, os.path.abspath(__file__), "--trace-pass", "--workload", args.workload,
           "--chain-ms", args.chain_ms, "--ms", args.ms]
    if args.only:
        cmd += ["--only", args.only]
    for flag in ("no_cells", "no_dependent", "no_probe"):
        if getattr(args, flag):
            cmd.append("--" + flag.replace("_", "-"))
    env = dict(os.environ, TMPDIR="/tmp")
    log("kernel trace: " + " ".join(cmd))
    t0 = time.perf_counter()
    try:
        # the child's stdout goes to our stderr: our stdout carries one JSON line only
        res = subprocess.run(cmd, cwd="/tmp", env=env, stdout=sys.stderr, stderr=sys.stderr,
                             timeout=900)
        rc = res.returncode
    except subprocess.TimeoutExpired:
        rc = "timeout"
    traces = sorted(glob.glob(os.path.join(out_dir, "**", "*kernel_trace.csv"), recursive=True))
    log(f"kernel trace: child exit {rc} after {time.perf_counter() - t0:.0f} s, {len(traces)} trace file(s)")
    if not traces:
        return None, f"no kernel trace (child exit {rc})"
    segs = split_trace(read_kernel_trace(traces), expected_trace_units(args))
    if not args.trace_dir:
        shutil.rmtree(out_dir, ignore_errors=True)
    return segs, f"child exit {rc}, {len(segs)} units traced"


# ---------------------------------------------------------------------------
# parity and CPU oracle
# ---------------------------------------------------------------------------

def check_output(ctx, y_dev, xb, wb, nthreads, repeats):
    """Oracle on the whole output (G1 per element, G2 per row, S1); returns
    (acceptance dict, oracle seconds: median of `repeats` runs)."""
    import oracle

    times, res = [], None
    for _ in range(max(1, repeats)):
        t1 = time.perf_counter()
        yr, ref, mag = oracle.gemm(xb, wb, nthreads=nthreads)
        times.append(time.perf_counter() - t1)
        if res is None and y_dev is not None:
            res = oracle.acceptance(ctx.to_host(y_dev), yr, ref, mag)
    return res, statistics.median(times)


def summarise_parity(results):
    ok = all(r["pass"] for r in results)
    return {"pass": bool(ok), "outputs_checked": len(results),
            "elements": int(sum(r["n"] for r in results)),
            "max_g1_ratio": round(max(r["max_g1_ratio"] for r in results), 4),
            "max_s1_ratio": round(max(r["max_s1_ratio"] for r in results), 4),
            "min_row_cosine": min(r["min_cos"] for r in results)}


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def time_chain_units(ctx, units, state, args, trace, want_parity, want_cpu):
    """The chain: the headline step (chain at the first M), the other Ms, the
    per-shape graphs, parity of every call's output and the CPU oracle."""
    import oracle

    torch = ctx.torch
    chains, headline = [], None
    by_name = {u.name: u for u in units}
    nthreads = oracle.default_threads()
    for M in chain_ms(args):
        u = by_name[f"chain:M{M}"]
        for _ in range(args.warmup):
            u.graph.replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for _ in range(args.steps):
            u.graph.replay()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = start.elapsed_time(end) / args.steps
        gbps, frac = rate(u.nbytes, ms * 1e3)
        log(f"chain M={M}: {ms:.4f} ms per step of {u.launches} calls, {gbps} GB/s "
            f"({100 * frac:.1f}% of 8 TB/s); wall {wall:.3f} s for {args.steps} steps")
        row = {"M": M, "ms_per_step": round(ms, 5), "us_per_call": round(ms * 1e3 / u.launches, 3),
               "gbps": gbps, "frac_of_peak": frac, "bytes_per_step": u.nbytes, "calls": u.launches,
               "wall_s": round(wall, 3), "groups": []}
        tr = trace.get(u.name) if trace else None
        if tr:
            row["kernel_us_sum_per_step"] = round(sum(tr) / TRACE_REPLAYS["chain"], 2)
        for (N, K, count) in CHAIN:
            g = by_name.get(f"group:({N},{K})M{M}")
            cell = (N, K, M)
            p, tuned, kname = plan_of(ctx, cell)
            grow = {"shape": f"({N},{K})", "calls": count, "kernel": kname, "plan": p.as_dict(),
                    "tuned_plan": tuned, "bytes_per_call": bytes_per_call(cell)}
            if g is not None:
                per = ctx.time_graph(g.graph, args.trials, max(10, args.replays // 3))
                us = statistics.median(per) / count
                grow["event_us_per_call"] = round(us, 3)
                grow["event_gbps"], grow["event_frac"] = rate(bytes_per_call(cell), us)
            if tr:
                first = g.meta["first"] if g is not None else sum(c for (n_, k_, c) in CHAIN[:CHAIN.index((N, K, count))])
                d = [tr[r * u.launches + first + i] for r in range(TRACE_REPLAYS["chain"]) for i in range(count)]
                grow["kernel"] = kname
                grow["rocprof"] = dist(d)
                grow["kernel_gbps"], grow["kernel_frac"] = rate(bytes_per_call(cell), statistics.mean(d))
            row["groups"].append(grow)
        # parity of every call's output, and the oracle's time per call
        if want_parity or (want_cpu and M == chain_ms(args)[0]):
            run = state["runs"][M]
            results, cpu_s = [], 0.0
            reps = 3 if (want_cpu and M == chain_ms(args)[0]) else 1
            for i, (N, K) in enumerate(CHAIN_CALLS):
                wb = ctx.to_host(state["weights"][i])
                res, s = check_output(ctx, run["ys"][i] if want_parity else None, run["xb"][K], wb,
                                      nthreads, reps)
                cpu_s += s
                if res is not None:
                    results.append(res)
            if results:
                row["parity"] = summarise_parity(results)
                log(f"chain M={M} parity: {row['parity']}")
            row["cpu_oracle_s_per_step"] = round(cpu_s, 3)
            row["cpu_oracle_repeats_per_call"] = reps
        chains.append(row)
        if headline is None:
            headline = row
    return chains, headline


def time_cell_units(ctx, units, state, args, trace, want_parity, want_cpu):
    import oracle

    rows = []
    nthreads = oracle.default_threads()
    deps = {u.name[4:]: u for u in units if u.kind == "dep"}
    for u in units:
        if u.kind != "cell":
            continue
        cell = u.meta["cell"]
        M = cell[-1]
        per = ctx.time_graph(u.graph, args.trials, args.replays)
        us = statistics.median(per) / u.launches
        b = bytes_per_call(cell)
        p, tuned, kname = plan_of(ctx, cell)
        row = {"cell": cell_name(cell), "bytes_per_call": b, "weight_bytes": weight_bytes(cell),
               "copies": u.launches, "kernel": kname, "plan": p.as_dict(), "tuned_plan": tuned,
               "replay_us_per_call": round(us, 3),
               "replay_us_min": round(min(per) / u.launches, 3),
               "replay_us_max": round(max(per) / u.launches, 3)}
        row["replay_gbps"], row["replay_frac"] = rate(b, us)
        tr = trace.get(u.name) if trace else None
        if tr:
            row["rocprof"] = dist(tr)
            row["kernel_us"] = row["rocprof"]["avg_us"]
            row["kernel_gbps"], row["kernel_frac"] = rate(b, row["kernel_us"])
            row["kernel_weight_gbps"] = rate(weight_bytes(cell), row["kernel_us"])[0]
        d = deps.get(cell_name(cell))
        if d is not None:
            dper = ctx.time_graph(d.graph, args.trials, max(10, args.replays // 3))
            row["dependent_us_per_call"] = round(statistics.median(dper) / d.launches, 3)
            dtr = trace.get(d.name) if trace else None
            if dtr:
                row["dependent_kernel_us"] = round(statistics.mean(dtr), 3)
        if args.vendor:
            row["vendor_us_per_call"] = round(time_vendor(ctx, state, M, cell, args), 3)
            row["speedup_vs_vendor"] = round(row["vendor_us_per_call"] / us, 3)
        run = state["runs"][M]
        if want_parity or want_cpu:
            reps = 3 if want_cpu else 1
            if cell[0] == "pair":
                res0, s0 = check_output(ctx, run["y"][0] if want_parity else None, run["xb"],
                                        state["host_w"][0], nthreads, reps)
                res1, s1 = check_output(ctx, run["y"][1] if want_parity else None, run["xb"],
                                        state["host_w"][1], nthreads, reps)
                results, cpu_s = [r for r in (res0, res1) if r is not None], s0 + s1
            else:
                res, cpu_s = check_output(ctx, run["y"] if want_parity else None, run["xb"],
                                          state["host_w"], nthreads, reps)
                results = [res] if res is not None else []
            if results:
                row["parity"] = summarise_parity(results)
            if want_cpu:
                row["cpu_oracle_us"] = round(cpu_s * 1e6, 1)
                row["cpu_oracle_gbps"] = round(b / cpu_s / 1e9, 3)
        log(f"cell {row['cell']}: kernel {row.get('kernel_us', 'n/a')} us "
            f"({100 * row.get('kernel_frac', 0):.1f}% of 8 TB/s), replay {us:.3f} us/call, "
            f"dependent {row.get('dependent_us_per_call', 'n/a')} us/call, "
            f"parity {row.get('parity', {}).get('pass', 'n/a')}")
        rows.append(row)
    return rows


def time_vendor(ctx, state, M, cell, args):
    """torch.nn.functional.linear on the same inputs and copies, same protocol (informational)."""
    lin = ctx.torch.nn.functional.linear
    run = state["runs"][M]

    def go():
        for w in run["ws"]:
            if cell[0] == "pair":
                lin(run["x"], w[0])
                lin(run["x"], w[1])
            else:
                lin(run["x"], w)
    g = ctx.capture(go)
    per = ctx.time_graph(g, args.trials, max(10, args.replays // 3))
    del g
    return statistics.median(per) / len(run["ws"])


def time_floor_units(ctx, units, args, trace):
    """Per weight size: the fastest probe shape (event and kernel-trace figures);
    per grid: the empty kernel's time per launch."""
    probes, empties = {}, []
    for u in units:
        if u.kind == "probe":
            per = ctx.time_graph(u.graph, args.trials, max(10, args.replays // 3))
            us = statistics.median(per) / u.launches
            rec = {"loads": u.meta["loads"], "threads": u.meta["threads"], "replay_us": round(us, 3)}
            tr = trace.get(u.name) if trace else None
            if tr:
                rec["kernel_us"] = round(statistics.mean(tr), 3)
            probes.setdefault(u.meta["size"], []).append(rec)
        elif u.kind == "empty":
            per = ctx.time_graph(u.graph, args.trials, 3)
            rec = {"grid": u.meta["grid"], "threads": 256,
                   "replay_us_per_launch": round(statistics.median(per) / u.launches, 3)}
            tr = trace.get(u.name) if trace else None
            if tr:
                rec["kernel_us"] = round(statistics.mean(tr), 3)
            empties.append(rec)
            log(f"empty kernel grid {rec['grid']}: {rec['replay_us_per_launch']} us per launch "
                f"(kernel {rec.get('kernel_us', 'n/a')} us)")
    reads = []
    for nb, recs in sorted(probes.items()):
        best_r = min(recs, key=lambda r: r["replay_us"])
        row = {"bytes": nb, "shapes": [str(s) for s in probe_sizes()[nb]],
               "best_replay": best_r, "all": recs}
        row["replay_gbps"] = rate(nb, best_r["replay_us"])[0]
        with_k = [r for r in recs if "kernel_us" in r]
        if with_k:
            best_k = min(with_k, key=lambda r: r["kernel_us"])
            row["best_kernel"] = best_k
            row["kernel_gbps"] = rate(nb, best_k["kernel_us"])[0]
        log(f"read probe {nb / 1e6:.1f} MB: replay {best_r['replay_us']} us "
            f"({row['replay_gbps']} GB/s), kernel {row.get('best_kernel', {}).get('kernel_us', 'n/a')} us")
        reads.append(row)
    return reads, empties


def attach_read_fractions(cells, reads):
    """Each cell's time as a fraction of the same-size read probe's (the probe
    reads the weight bytes only)."""
    by_size = {r["bytes"]: r for r in reads}
    for c in cells:
        r = by_size.get(c["weight_bytes"])
        if r is None:
            continue
        c["read_probe_replay_us"] = r["best_replay"]["replay_us"]
        c["replay_vs_read"] = round(r["best_replay"]["replay_us"] / c["replay_us_per_call"], 4)
        if "best_kernel" in r and "kernel_us" in c:
            c["read_probe_kernel_us"] = r["best_kernel"]["kernel_us"]
            c["kernel_vs_read"] = round(r["best_kernel"]["kernel_us"] / c["kernel_us"], 4)


def dominant_kernel(chain_row):
    """The compiled kernel instance with the largest share of the headline step,
    the chain's shapes pooled by kernel name (as rocprofv3 --stats aggregates)."""
    pooled = {}
    for g in chain_row["groups"]:
        if "event_us_per_call" not in g:
            continue
        p = pooled.setdefault(g["kernel"], {"us": 0.0, "launches": 0, "bytes": 0, "shapes": [],
                                            "rocprof_us": 0.0, "rocprof_n": 0})
        p["us"] += g["event_us_per_call"] * g["calls"]
        p["launches"] += g["calls"]
        p["bytes"] += g["bytes_per_call"] * g["calls"]
        p["shapes"].append(g["shape"])
        if "rocprof" in g:
            p["rocprof_us"] += g["rocprof"]["avg_us"] * g["calls"]
            p["rocprof_n"] += g["calls"]
    if not pooled:
        return None
    name, d = max(pooled.items(), key=lambda kv: kv[1]["us"])
    avg = d["us"] / d["launches"]
    bpl = d["bytes"] / d["launches"]
    achieved = bpl / (avg * 1e-6) / 1e9
    out = {"bound": "hbm", "kernel": name, "shapes": d["shapes"], "M": chain_row["M"],
           "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
           "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": recorded_traffic("chain", name),
           "avg_launch_us": round(avg, 3), "launches_per_step": d["launches"],
           "algorithmic_bytes_per_launch": round(bpl),
           "share_of_step": round(d["us"] / sum(p["us"] for p in pooled.values()), 4)}
    if d["rocprof_n"] == d["launches"]:
        ra = d["rocprof_us"] / d["rocprof_n"]
        out["rocprof_avg_launch_us"] = round(ra, 3)
        out["rocprof_frac"] = round(bpl / (ra * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
    return out


def dominant_cell_kernel(cells, workload):
    pooled = {}
    for c in cells:
        p = pooled.setdefault(c["kernel"], {"us": 0.0, "launches": 0, "bytes": 0, "cells": []})
        p["us"] += c["replay_us_per_call"] * c["copies"]
        p["launches"] += c["copies"]
        p["bytes"] += c["bytes_per_call"] * c["copies"]
        p["cells"].append(c["cell"])
    name, d = max(pooled.items(), key=lambda kv: kv[1]["us"])
    avg = d["us"] / d["launches"]
    bpl = d["bytes"] / d["launches"]
    achieved = bpl / (avg * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": name, "cells": d["cells"], "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": recorded_traffic(workload, name), "avg_launch_us": round(avg, 3),
            "launches_per_step": d["launches"], "algorithmic_bytes_per_launch": round(bpl),
            "share_of_step": round(d["us"] / sum(p["us"] for p in pooled.values()), 4)}


def main(argv=None) -> int:
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. "
              "The GEMV shards by output rows with no exchange, so N GPUs each run one "
              "rank's share at its own shape; run with --gpus 1.", file=sys.stderr)
        return 2
    if args.trace_pass:
        return trace_pass(args)
    if args.copy_calibration:
        return copy_calibration()
    if args.read_probe:
        args.no_cells, args.workload = True, "chain"

    # the kernel-trace child runs first, before this process touches the GPU
    trace, trace_note = None, "skipped (--no-trace)"
    if args.read_probe:
        trace_note = "skipped (--read-probe)"
    elif not args.no_trace:
        if under_profiler():
            trace_note = "skipped: this process already runs under a profiler"
        else:
            trace, trace_note = run_trace_child(args)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    ctx = Ctx(args)
    props = torch.cuda.get_device_properties(ctx.dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")
    want_parity, want_cpu = not args.no_parity, not args.no_cpu

    if args.read_probe:
        units, _ = floor_group(ctx)
        reads, empties = time_floor_units(ctx, units, args, None)
        print(json.dumps({"read_probe": reads, "empty_kernel": empties}), flush=True)
        return 0

    cells_sel, with_chain = traced_units(args)
    chains, headline, cells, reads, empties = [], None, [], [], []
    # a cell workload's step replays every cell's graph: their buffers stay referenced
    step_units, step_states = [], []
    for gname, units, state in unit_groups(ctx, cells_sel, with_chain, True, not args.no_dependent,
                                           not args.no_probe):
        log(f"group {gname}: {len(units)} graphs captured")
        if gname == "chain":
            chains, headline = time_chain_units(ctx, units, state, args, trace, want_parity, want_cpu)
        elif gname == "floor":
            reads, empties = time_floor_units(ctx, units, args, trace)
        else:
            cells += time_cell_units(ctx, units, state, args, trace, want_parity, want_cpu)
            if not with_chain:
                step_units += [u for u in units if u.kind == "cell"]
                step_states.append(state)
                continue
        del units, state
    attach_read_fractions(cells, reads)

    nt = None
    if want_cpu:
        import oracle

        nt = oracle.default_threads()
    if with_chain:
        value, ms_per_step = headline["gbps"], headline["ms_per_step"]
        roofline = dominant_kernel(headline)
        cpu = None
        if want_cpu and "cpu_oracle_s_per_step" in headline:
            s = headline["cpu_oracle_s_per_step"]
            cpu = {"value": round(headline["bytes_per_step"] / s / 1e9, 3), "unit": "GB/s", "cores": nt,
                   "kind": "oracle", "cpu_model": cpu_model(),
                   "sample": f"the whole M={headline['M']} decode-step chain: each of the 186 calls "
                             f"run through the fp64 C oracle on a host copy of its weight, one weight "
                             f"at a time, median of {headline['cpu_oracle_repeats_per_call']} runs per "
                             f"call, summed: {s:.2f} s per step ({s * 1e3 / 186:.2f} ms per call)"}
        config = {"workload": CHAIN_DESC + f", M={headline['M']}", "M": headline["M"],
                  "launches_per_step": headline["calls"], "bytes_per_step": headline["bytes_per_step"],
                  "accumulate": "fp32", "device": props.name, "source_digest": source_digest()}
    else:
        # the step: every cell of the workload once over its copies
        for _ in range(args.warmup):
            for u in step_units:
                u.graph.replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            for u in step_units:
                u.graph.replay()
        end.record()
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(end) / args.steps
        step_bytes = sum(u.nbytes for u in step_units)
        value = round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2)
        roofline = dominant_cell_kernel(cells, args.workload)
        cpu = None
        if want_cpu and all("cpu_oracle_us" in c for c in cells):
            s = sum(c["cpu_oracle_us"] * 1e-6 for c in cells)
            cpu = {"value": round(sum(c["bytes_per_call"] for c in cells) / s / 1e9, 3), "unit": "GB/s",
                   "cores": nt, "kind": "oracle", "cpu_model": cpu_model(),
                   "sample": f"one call of each of the {len(cells)} cells, fp64 C oracle, median of 3 "
                             f"runs each, {s:.2f} s"}
        desc = (CELL_WORKLOADS[args.workload][0] if args.workload in CELL_WORKLOADS else
                "cells " + ", ".join(cell_name(shape_cell(sh, m)) for sh, ms in cells_sel for m in ms))
        config = {"workload": desc,
                  "launches_per_step": sum(u.launches for u in step_units), "bytes_per_step": step_bytes,
                  "rotation_bytes_min": ROTATE_BYTES, "accumulate": "fp32", "device": props.name,
                  "source_digest": source_digest()}

    parity_parts = [c["parity"] for c in chains if "parity" in c] + [c["parity"] for c in cells if "parity" in c]
    parity = None
    if parity_parts:
        parity = {"pass": all(p["pass"] for p in parity_parts),
                  "outputs_checked": sum(p["outputs_checked"] for p in parity_parts),
                  "elements": sum(p["elements"] for p in parity_parts),
                  "max_g1_ratio": max(p["max_g1_ratio"] for p in parity_parts),
                  "max_s1_ratio": max(p["max_s1_ratio"] for p in parity_parts),
                  "min_row_cosine": min(p["min_row_cosine"] for p in parity_parts),
                  "sampled": False}
    out = {
        "metric": METRIC,
        "value": value,
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
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "chains": chains,
        "cells": cells,
        "read_probe": reads,
        "empty_kernel": empties,
        "kernel_trace": trace_note,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
