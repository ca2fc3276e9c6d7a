"""On-device plan sweep for the skinny GEMM plan table.

For each (N, K, M) it times every compiled variant that can run the shape,
at several block sizes and with both grid modes (persistent, one block per
tile), and keeps the fastest. This follows the method of vLLM PR #62949 (SM121
skinny GEMM plans), section Details (a graph-replay sweep over the plan knobs
with the weight rotated out of the cache) and vLLM PR #65306 (SM90 skinny GEMM
plans), section Validation (a graph-captured chain over weight copies of at
least 1 GiB, timed in trials of replays), with the copies sized past the
MI355X's 256 MB Infinity Cache.

    python -m bf16_skinny_gemm_amd.sweep --out sweep.jsonl          # measure (GPU)
    python -m bf16_skinny_gemm_amd.sweep --emit-inc sweep.jsonl      # write plans_gfx950.inc

Measurements are appended one JSON line per (cell, plan); a rerun skips cells
already complete in the output file, so an interrupted sweep resumes.

Every cell starts with one untimed graph replay cycle: the first plan timed after
the weight copies are written otherwise reads several percent slow. With
--rounds R > 1 the --finalists fastest plans of the single pass are timed R more
times, the order rotated every round, and their records (stage 2, median of the
rounds) are the only ones the table generator considers for that cell.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
INC_PATH = os.path.join(HERE, "csrc", "plans_gfx950.inc")
ROTATE_BYTES = 1 << 30

# The decode projections at M = 1, 2, 4 (and 3, which the API supports): the TP=2
# rank shapes of vLLM PR #62949 (section Validation), the TP4/TP8 rank shapes of
# vLLM PR #65306 (section Validation: LM head / KDA in_proj rows (6416, 4096),
# (19360, 4096), (38720, 4096)) and the router gate (288, 4096) (float32 output; it
# shares the bf16 plan). Paired f_b/g_b weights (4096, 128) and the TP4 pair
# (2048, 128) are swept as pairs.
SHAPES = [(4096, 1024), (12576, 4096), (4096, 4096), (2048, 4096), (8192, 1536), (4096, 8192),
          (77440, 4096), (6416, 4096), (19360, 4096), (38720, 4096), (288, 4096), (256, 4096)]
PAIR_SHAPES = [(4096, 128), (2048, 128)]
MS = (1, 2, 3, 4, 5, 6, 7, 8)
BIG_GRID = 1 << 30  # grid_blocks >= tile count: one block per tile
SAME = -2           # grid token: the grid a refined variant had in its fastest record
BALANCED = -1       # grid token: block counts that give every block the same tile count
PLAN_FIELDS = ("kind", "threads_per_block", "lanes_per_row", "chunks", "rows_per_wave", "k_split",
               "nontemporal", "grid_blocks", "x_in_lds", "prefetch")


def log(msg):
    print(f"[sweep {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse_grids(spec: str) -> tuple:
    """Grid modes from a comma list: 'persistent' (0: one resident wave of blocks),
    'tile' (one block per tile), a block count (a persistent grid of at most
    that many blocks), and for --refine 'same' (SAME) and 'balanced' (BALANCED)."""
    named = {"persistent": 0, "tile": BIG_GRID, "same": SAME, "balanced": BALANCED}
    out = []
    for g in spec.split(","):
        g = g.strip()
        out.append(named[g] if g in named else int(g))
    return tuple(out)


def rows_per_tile(d) -> int | None:
    """Output rows a block covers per tile under plan dict d (as the library's
    launcher computes them), or None for the element-wise kind."""
    waves = d["threads_per_block"] // 64
    if d["kind"] == 1:
        per_group = d["rows_per_wave"] * (64 // d["lanes_per_row"])
    elif d["kind"] == 2:
        per_group = d["rows_per_wave"]
    elif d["kind"] == 4:
        per_group = 4 * d["rows_per_wave"]
    else:
        return None
    return (waves // d["k_split"]) * per_group


def balanced_grids(d, N, nmats=1, near=None, count=4, lo=128, hi=4096) -> list:
    """Grids (grid_blocks values) under which every block of plan d takes the same
    number of tiles, or all but one do: ceil(T / t) blocks for t tiles per block,
    T = ceil(N / rows per tile). A grid of 512 blocks over 3144 tiles leaves 72
    blocks with a 7th tile while the rest stop at 6; 524 or 450 blocks do not.
    The `count` nearest to `near` blocks per weight (default: d's own explicit
    grid, else 512) are returned, times nmats for a pair."""
    rpt = rows_per_tile(d)
    if rpt is None:
        return []
    tiles = -(-N // rpt)
    if near is None:
        g0 = d["grid_blocks"] // nmats
        near = g0 if 0 < g0 < BIG_GRID // 2 else 512
    out = []
    for t in range(1, tiles + 1):
        g = -(-tiles // t)
        if g < lo:
            break
        if g <= hi and g < tiles and g not in out:
            out.append(g)
    out.sort(key=lambda g: (abs(math.log(g / near)), g))
    return [g * nmats for g in out[:count]]


def table_plans(path: str = INC_PATH) -> dict:
    """The plan table as {(N, K, M): plan dict}, read back from its .inc file."""
    out = {}
    row = re.compile(r"^\{(\d+), (\d+), (\d+), \{([-\d, ]+)\}\},")
    with open(path) as f:
        for line in f:
            m = row.match(line)
            if m:
                vals = [int(v) for v in m.group(4).split(",")]
                out[(int(m.group(1)), int(m.group(2)), int(m.group(3)))] = dict(zip(PLAN_FIELDS, vals))
    return out


def rotated_order(n: int, rnd: int) -> list:
    """Timing order of n plans in round rnd: plan rnd mod n first, then the others
    onwards (even rounds) or backwards (odd rounds), so that no plan is always
    timed first or right after the same neighbour."""
    if n == 0:
        return []
    k = rnd % n
    rest = [(k + i) % n for i in range(1, n)]
    return [k] + (rest[::-1] if rnd % 2 else rest)


def split_k_plans(skg, K, M, N):
    """Every cross-block split-K plan able to run (K, M): each compiled variant at
    the slice count that makes K, block sizes 64..512."""
    out = []
    for v in skg.split_k_variants():
        d = v.as_dict()
        slice_k = d["lanes_per_row"] * 8 * d["chunks"]
        if K % slice_k or K // slice_k > 16:
            continue
        for tpb in (64, 128, 256, 512):
            p = skg.Plan.from_dict({**d, "threads_per_block": tpb, "k_split": K // slice_k})
            if skg.skinny_gemm_split_k_workspace_bytes(M, N, K, p):
                out.append(p)
    return out


def candidate_plans(skg, K, M, kinds=None, grids=(0, BIG_GRID)):
    """Every (variant, block size, grid mode) able to run (K, M)."""
    out = []
    for v in skg.variants():
        d = v.as_dict()
        if d["kind"] == skg.SKINNY_KIND_SCALAR or (kinds and d["kind"] not in kinds):
            continue
        if d["kind"] == skg.SKINNY_KIND_FIXED_K and \
                d["k_split"] * d["lanes_per_row"] * 8 * d["chunks"] != K:
            continue
        if d["kind"] == skg.SKINNY_KIND_MFMA and \
                (K % (128 * d["k_split"]) or (K // (128 * d["k_split"])) % d["chunks"]):
            continue
        for tpb in (128, 256, 512):
            if (tpb // 64) % d["k_split"]:
                continue
            for grid in grids:
                out.append(skg.Plan.from_dict({**d, "threads_per_block": tpb, "grid_blocks": grid}))
    return out


def plan_key(p) -> tuple:
    d = p.as_dict()
    return tuple(d[k] for k in PLAN_FIELDS)


def time_plan(torch, skg, x, weights, ys, plan, pair, trials, replays):
    """Median microseconds per call over graph replays of one call per weight copy."""
    ws = None
    if plan.kind == skg.SKINNY_KIND_SPLIT_K:  # one workspace serves the calls in turn
        ws = skg.split_k_workspace(x.shape[0], weights[0].shape[0], x.shape[1], plan, device=x.device)

    def run():
        for w in weights:
            if ws is not None:
                skg.gemm_split_k(x, w, ws, plan=plan, out=ys)
            elif pair:
                skg.gemm_pair(x, w[0], w[1], out0=ys[0], out1=ys[1], plan=plan)
            else:
                skg.gemm(x, w, out=ys, plan=plan)

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
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / (replays * len(weights)))
    del g
    return statistics.median(per), min(per), max(per)


def done_keys(path):
    keys = set()
    if os.path.exists(path):
        with open(path) as f:
            for line in f:
                try:
                    r = json.loads(line)
                except json.JSONDecodeError:
                    continue
                if r.get("complete"):
                    keys.add((r["N"], r["K"], r["M"], r["pair"]))
    return keys


def lookahead_twin(d, M):
    """The same fixed-K plan with x in LDS read one chunk ahead (x_in_lds 2), for
    plans with one row per wave at M >= 2 (the only ones compiled), else None."""
    if d["kind"] != 1 or d["rows_per_wave"] != 1 or d["x_in_lds"] == 2 or M < 2:
        return None
    return {**d, "x_in_lds": 2}


def refine_plans(skg, path, N, K, M, pair, top, grids, twins=False):
    """The `top` fastest (variant, block size) pairs of a cell in earlier sweep
    files (a comma list, records pooled), each crossed with `grids`, where SAME is
    the grid of the pair's fastest record and BALANCED expands to balanced_grids()
    near it; with grids None, the `top` fastest plans as they are (grid included),
    to re-time the close contenders with more replays. With `twins`, each plan's
    lookahead twin (lookahead_twin) is timed after it."""
    recs = []
    for one in path.split(","):
        with open(one) as f:
            for line in f:
                r = json.loads(line)
                if "plan" in r and (r["N"], r["K"], r["M"], r["pair"]) == (N, K, M, pair):
                    recs.append(r)
    recs.sort(key=lambda r: r["us"])
    if grids is None:
        dicts = [r["plan"] for r in recs[:top]]
    else:
        nmats = 2 if pair else 1
        seen, dicts = set(), []
        for r in recs:
            d = {k: v for k, v in r["plan"].items() if k != "grid_blocks"}
            key = tuple(sorted(d.items()))
            if key in seen:
                continue
            seen.add(key)
            own = r["plan"]["grid_blocks"]
            for g in grids:
                if g == SAME:
                    dicts.append({**d, "grid_blocks": own})
                elif g == BALANCED:
                    dicts.extend({**d, "grid_blocks": b}
                                 for b in balanced_grids(r["plan"], N, nmats))
                else:
                    dicts.append({**d, "grid_blocks": g})
            if len(seen) >= top:
                break
    out, keys = [], set()
    for d in dicts:
        for cand in (d, lookahead_twin(d, M) if twins else None):
            if cand is None:
                continue
            key = tuple(sorted(cand.items()))
            if key not in keys:
                keys.add(key)
                out.append(skg.Plan.from_dict(cand))
    return out


def measure(args):
    import torch

    import bf16_skinny_gemm_amd as skg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    skg.skinny_gemm_init(0)
    done = done_keys(args.out)
    if args.shapes:
        cells = [tuple(int(v) for v in sh.split("x")) + (False,) for sh in args.shapes.split(",")]
    else:
        cells = [(N, K, False) for (N, K) in SHAPES] + [(N, K, True) for (N, K) in PAIR_SHAPES]
    if args.only:
        want = {tuple(int(v) for v in s.split("x")) for s in args.only.split(",")}
        cells = [c for c in cells if (c[0], c[1]) in want]
    ms = tuple(int(m) for m in args.ms.split(","))
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    table = table_plans(args.inc_path) if args.with_table else {}
    t_start = time.monotonic()

    def out_of_time():
        if args.budget and time.monotonic() - t_start > args.budget:
            log(f"time budget of {args.budget:.0f} s spent: stopping; rerun to resume")
            return True
        return False

    with open(args.out, "a") as fout:
        for (N, K, pair) in cells:
            todo = [M for M in ms if (N, K, M, pair) not in done]
            if not todo:
                continue
            if out_of_time():
                break
            wbytes = (4 if pair else 2) * N * K
            copies = max(2, math.ceil(ROTATE_BYTES / wbytes))
            base = (torch.randn((N, K), generator=gen, device=dev) / math.sqrt(K)).to(torch.bfloat16)
            if pair:
                base1 = (torch.randn((N, K), generator=gen, device=dev) / math.sqrt(K)).to(torch.bfloat16)
                weights = [(base, base1)] + [(base.clone(), base1.clone()) for _ in range(copies - 1)]
            else:
                weights = [base] + [base.clone() for _ in range(copies - 1)]
            log(f"shape ({N},{K}) pair={pair}: {copies} copies")
            for M in todo:
                if out_of_time():
                    break
                x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
                ys = ((torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                       torch.empty((M, N), dtype=torch.bfloat16, device=dev)) if pair
                      else torch.empty((M, N), dtype=torch.bfloat16, device=dev))
                nbytes = (4 * N * K + 2 * M * K + 4 * M * N) if pair else (2 * N * K + 2 * M * K + 2 * M * N)
                best = None
                kinds = {int(k) for k in args.kinds.split(",")} if args.kinds else None
                grids = None if args.grids == "same" else parse_grids(args.grids)
                if kinds == {skg.SKINNY_KIND_SPLIT_K}:
                    plans = [] if pair else split_k_plans(skg, K, M, N)
                else:
                    plans = (refine_plans(skg, args.refine, N, K, M, pair, args.top, grids, args.twins)
                             if args.refine else candidate_plans(skg, K, M, kinds, grids))
                current = None
                if args.with_table:
                    # the table's plan for the cell (for a shape the table does not hold,
                    # the library's default plan) runs first and is always a finalist, so
                    # a new plan replaces it only by beating it in the same rounds
                    if (N, K, M) in table:
                        current = skg.Plan.from_dict(table[(N, K, M)])
                    elif not pair:
                        current = skg.skinny_gemm_get_plan(N, K, M)[0]
                    if current is not None:
                        plans = [current] + [p for p in plans if plan_key(p) != plan_key(current)]
                staged = args.rounds > 1

                def record(plan, us, lo, hi, stage):
                    rec = {"N": N, "K": K, "M": M, "pair": pair, "plan": plan.as_dict(),
                           "us": round(us, 4), "us_min": round(lo, 4), "us_max": round(hi, 4),
                           "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
                    if staged:
                        rec["stage"] = stage
                    if current is not None and plan_key(plan) == plan_key(current):
                        rec["incumbent"] = True
                    fout.write(json.dumps(rec) + "\n")

                warmed = False
                timed = []
                for plan in plans:
                    try:
                        if not warmed:  # untimed: the first timing after the copies reads slow
                            time_plan(torch, skg, x, weights, ys, plan, pair, 1, 3)
                            warmed = True
                        us, lo, hi = time_plan(torch, skg, x, weights, ys, plan, pair,
                                               args.trials, args.replays)
                    except skg.SkinnyError:
                        continue  # this M does not fit the variant
                    record(plan, us, lo, hi, 1)
                    timed.append((us, plan))
                if staged and timed:
                    finalists = [p for _, p in sorted(timed, key=lambda t: t[0])[:args.finalists]]
                    if current is not None and all(plan_key(p) != plan_key(current) for p in finalists):
                        finalists[-1] = current
                    rounds = [[] for _ in finalists]
                    for rnd in range(args.rounds):
                        for i in rotated_order(len(finalists), rnd):
                            us, _, _ = time_plan(torch, skg, x, weights, ys, finalists[i], pair,
                                                 args.trials, args.replays)
                            rounds[i].append(us)
                    timed = []
                    for plan, v in zip(finalists, rounds):
                        record(plan, statistics.median(v), min(v), max(v), 2)
                        timed.append((statistics.median(v), plan))
                for us, plan in timed:
                    if best is None or us < best[0]:
                        best = (us, plan)
                fout.write(json.dumps({"N": N, "K": K, "M": M, "pair": pair, "complete": True}) + "\n")
                fout.flush()
                if best is None:
                    log(f"  M={M}: no plan ran")
                    continue
                log(f"  M={M}: best {best[0]:.3f} us {nbytes / (best[0] * 1e-6) / 1e9:.0f} GB/s {best[1]}")
            del weights, base
            torch.cuda.empty_cache()


def pick(records, tol=0.005):
    """Fastest plan; within `tol` of it prefer the persistent grid, no cache hint,
    fewer rows per wave, smaller blocks (simpler, more robust to other shapes)."""
    best_us = min(r["us"] for r in records)
    near = [r for r in records if r["us"] <= best_us * (1 + tol)]
    near.sort(key=lambda r: (r["plan"]["grid_blocks"] != 0, r["plan"]["nontemporal"],
                             r["plan"]["rows_per_wave"], r["plan"]["threads_per_block"], r["us"]))
    return near[0]


def emit_inc(paths, out=INC_PATH):
    """Write the plan table from one or more sweep files. A cell's records come
    from the last file in the list that holds the cell, so a later pass over
    some cells (timed on one box, in the same rounds) replaces the earlier one
    for those cells without mixing timings from different runs."""
    recs = {}
    for path in paths.split(","):
        mine = {}
        with open(path) as f:
            for line in f:
                r = json.loads(line)
                if "plan" not in r or r["plan"]["kind"] == 5:  # split-K: not for the table
                    continue
                mine.setdefault((r["N"], r["K"], r["M"]), []).append(r)
        recs.update(mine)
    for key, rs in recs.items():
        # a cell re-timed in rounds is decided by those records alone
        if any(r.get("stage") == 2 for r in rs):
            recs[key] = [r for r in rs if r.get("stage") == 2]
    lines = [
        "// Tuned launch plans for gfx950, one line per (N, K, M):",
        "//   {N, K, M, {kind, threads_per_block, lanes_per_row, chunks, rows_per_wave, k_split,",
        "//            nontemporal, grid_blocks, x_in_lds, prefetch}},",
        "// Generated by `python -m bf16_skinny_gemm_amd.sweep --emit-inc` from an on-device sweep",
        "// (MI355X, weights rotated over >= 1 GiB of copies, hipGraph replay). Do not edit by hand.",
    ]
    for (N, K, M) in sorted(recs):
        r = pick(recs[(N, K, M)])
        p = r["plan"]
        fields = ", ".join(str(p.get(k, 0)) for k in PLAN_FIELDS)
        lines.append(f"{{{N}, {K}, {M}, {{{fields}}}}},  // {r['us']:.3f} us, {r['gbps']:.0f} GB/s")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


def split_k_report(path) -> str:
    """Per cell of a `--kinds 5 --with-table` sweep: the table's plan against the
    fastest split-K plan, both from the same rounds (stage 2 when timed in rounds)."""
    by = {}
    with open(path) as f:
        for line in f:
            r = json.loads(line)
            if "plan" in r:
                by.setdefault((r["N"], r["K"], r["M"]), []).append(r)
    rows = ["| (N, K) | M | table plan µs | best split-K µs | split-K ÷ table | split-K plan "
            "(lanes, chunks, rows/wave, S, threads) |", "|---|---|---|---|---|---|"]
    for (N, K, M) in sorted(by):
        rs = by[(N, K, M)]
        final = [r for r in rs if r.get("stage") == 2] or rs
        table = [r for r in final if r["plan"]["kind"] != 5]
        split = [r for r in final if r["plan"]["kind"] == 5] or [r for r in rs if r["plan"]["kind"] == 5]
        if not table or not split:
            continue
        t = min(r["us"] for r in table)
        b = min(split, key=lambda r: r["us"])
        p = b["plan"]
        rows.append(f"| ({N},{K}) | {M} | {t:.3f} | {b['us']:.3f} | {b['us'] / t:.2f} | "
                    f"({p['lanes_per_row']}, {p['chunks']}, {p['rows_per_wave']}, {p['k_split']}, "
                    f"{p['threads_per_block']}) |")
    return "\n".join(rows)


def incumbent_report(path) -> str:
    """Per cell of a `--with-table` sweep: the incumbent plan (the table's, or the
    library's default for a shape the table does not hold) against the fastest plan
    timed, both from the same rounds (stage 2 when timed in rounds)."""
    by = {}
    with open(path) as f:
        for line in f:
            r = json.loads(line)
            if "plan" in r:
                by.setdefault((r["N"], r["K"], r["M"]), []).append(r)
    rows = ["| (N, K) | M | incumbent µs | best µs | incumbent ÷ best | best plan |", "|---|---|---|---|---|---|"]
    for (N, K, M) in sorted(by):
        rs = by[(N, K, M)]
        final = [r for r in rs if r.get("stage") == 2] or rs
        inc = [r for r in final if r.get("incumbent")]
        if not inc:
            continue
        b = min(final, key=lambda r: r["us"])
        p = b["plan"]
        desc = ", ".join(f"{k}={p[k]}" for k in PLAN_FIELDS)
        rows.append(f"| ({N},{K}) | {M} | {inc[0]['us']:.3f} | {b['us']:.3f} | {inc[0]['us'] / b['us']:.3f} | {desc} |")
    return "\n".join(rows)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", help="JSON-lines file to append measurements to")
    ap.add_argument("--emit-inc", metavar="JSONL[,JSONL...]",
                    help="write the plan table from sweep files (records pooled)")
    ap.add_argument("--inc-path", default=INC_PATH)
    ap.add_argument("--incumbent-report", metavar="JSONL",
                    help="print incumbent (table or default) plan vs fastest plan per cell of a --with-table sweep")
    ap.add_argument("--split-k-report", metavar="JSONL",
                    help="print table-plan vs split-K times per cell of a --kinds 5 --with-table sweep")
    ap.add_argument("--only", help="comma list of NxK shapes to sweep")
    ap.add_argument("--shapes", help="comma list of NxK shapes to sweep instead of the decode "
                    "projections (e.g. shapes outside the table, to rate the default plan)")
    ap.add_argument("--ms", default=",".join(str(m) for m in MS))
    ap.add_argument("--kinds", help="comma list of plan kinds to time (default: all)")
    ap.add_argument("--grids", default="persistent,tile",
                    help="comma list of grid modes: persistent, tile, or a block count; "
                         "with --refine, 'same' alone keeps each plan as it is, and in a "
                         "list 'same' is a variant's fastest grid and 'balanced' the grids "
                         "that give every block the same number of tiles")
    ap.add_argument("--refine", metavar="JSONL[,JSONL...]",
                    help="time only the --top fastest plans per cell of earlier sweeps, at --grids")
    ap.add_argument("--rounds", type=int, default=1,
                    help="re-time the --finalists fastest plans of each cell this many more "
                         "times, in rotated order; their medians decide the cell")
    ap.add_argument("--finalists", type=int, default=6)
    ap.add_argument("--with-table", action="store_true",
                    help="also time each cell's plan from the current table (--inc-path) and keep "
                         "it among the finalists")
    ap.add_argument("--top", type=int, default=16)
    ap.add_argument("--twins", action="store_true",
                    help="with --refine, also time each plan with x read from LDS one chunk ahead")
    ap.add_argument("--budget", type=float, default=0.0,
                    help="stop starting new cells after this many seconds (0: no limit)")
    ap.add_argument("--trials", type=int, default=3)
    ap.add_argument("--replays", type=int, default=5)
    args = ap.parse_args()
    if args.split_k_report:
        print(split_k_report(args.split_k_report))
        return 0
    if args.incumbent_report:
        print(incumbent_report(args.incumbent_report))
        return 0
    if args.emit_inc:
        print(emit_inc(args.emit_inc, args.inc_path))
        return 0
    if not args.out:
        ap.error("--out or --emit-inc is required")
    if not args.refine and args.grids != "same" and any(g < 0 for g in parse_grids(args.grids)):
        ap.error("grid modes 'same' and 'balanced' need --refine")
    measure(args)
    return 0


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(HERE))
    sys.exit(main())
