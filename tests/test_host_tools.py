"""Host-side logic of the plan sweep and the benchmark (no GPU needed)."""
from __future__ import annotations

import json
import os
import re

import pytest

import bench
from bf16_skinny_gemm_amd import sweep


def _rec(N, K, M, us, **plan):
    p = {"kind": 1, "threads_per_block": 256, "lanes_per_row": 64, "chunks": 4,
         "rows_per_wave": 1, "k_split": 2, "nontemporal": 1, "grid_blocks": 0, "x_in_lds": 0,
         "prefetch": 0}
    p.update(plan)
    return {"N": N, "K": K, "M": M, "pair": False, "plan": p, "us": us, "us_min": us,
            "us_max": us, "gbps": 1.0}


def test_parse_grids():
    assert sweep.parse_grids("persistent,tile,256, 512") == (0, sweep.BIG_GRID, 256, 512)


def test_pick_prefers_persistent_within_tolerance():
    tile = _rec(1, 8, 1, 10.00, grid_blocks=sweep.BIG_GRID)
    pers = _rec(1, 8, 1, 10.04, grid_blocks=0)
    assert sweep.pick([tile, pers])["plan"]["grid_blocks"] == 0      # within 0.5%
    slow = _rec(1, 8, 1, 10.20, grid_blocks=0)
    assert sweep.pick([tile, slow])["plan"]["grid_blocks"] == sweep.BIG_GRID


def test_emit_inc_one_row_per_cell(tmp_path):
    recs = [_rec(4096, 4096, 1, 7.0, chunks=8, k_split=1), _rec(4096, 4096, 1, 6.9),
            _rec(4096, 4096, 2, 7.5, prefetch=2, grid_blocks=512), {"N": 4096, "K": 4096,
                                                                     "M": 2, "complete": True}]
    src = tmp_path / "s.jsonl"
    src.write_text("".join(json.dumps(r) + "\n" for r in recs))
    out = tmp_path / "plans.inc"
    sweep.emit_inc(str(src), str(out))
    rows = re.findall(r"^\{(\d+), (\d+), (\d+), \{([^}]*)\}\},", out.read_text(), re.M)
    assert [(int(a), int(b), int(c)) for a, b, c, _ in rows] == [(4096, 4096, 1), (4096, 4096, 2)]
    fields = [int(v) for v in rows[0][3].split(",")]
    assert fields == [1, 256, 64, 4, 1, 2, 1, 0, 0, 0]               # the 6.9 us plan
    fields = [int(v) for v in rows[1][3].split(",")]
    assert fields[7] == 512 and fields[9] == 2


def test_refine_takes_top_variants_times_grids(tmp_path):
    import bf16_skinny_gemm_amd as skg

    recs = [_rec(100, 4096, 1, 5.0, grid_blocks=0), _rec(100, 4096, 1, 5.1, grid_blocks=256),
            _rec(100, 4096, 1, 6.0, chunks=8, k_split=1), _rec(100, 4096, 1, 7.0, prefetch=2),
            _rec(100, 4096, 2, 1.0, prefetch=1)]                     # other cell: ignored
    src = tmp_path / "s.jsonl"
    src.write_text("".join(json.dumps(r) + "\n" for r in recs))
    plans = sweep.refine_plans(skg, str(src), 100, 4096, 1, False, 2, (0, 512))
    got = [(p.chunks, p.k_split, p.prefetch, p.grid_blocks) for p in plans]
    assert got == [(4, 2, 0, 0), (4, 2, 0, 512), (8, 1, 0, 0), (8, 1, 0, 512)]


def test_kernel_names_follow_the_templates():
    import bf16_skinny_gemm_amd as skg

    p = skg.Plan.from_dict({"kind": 1, "threads_per_block": 256, "lanes_per_row": 64, "chunks": 8,
                            "rows_per_wave": 1, "k_split": 1, "nontemporal": 1, "grid_blocks": 0,
                            "x_in_lds": 1, "prefetch": 2})
    assert bench.kernel_name(p, 4) == \
        "void skg::fixed_k_kernel<4, 64, 8, 1, 1, 1, true, 2>(skg::Args)"
    p.kind, p.chunks, p.rows_per_wave = 2, 4, 2
    assert bench.kernel_name(p, 3) == "void skg::loop_k_kernel<3, 4, 2, true>(skg::Args, int)"
    p.kind, p.chunks, p.rows_per_wave, p.k_split, p.prefetch = 4, 2, 1, 4, 1
    assert bench.kernel_name(p, 1) == "void skg::mfma_kernel<1, 2, 1, 4, true, true>(skg::Args)"
    p.kind = 3
    assert bench.kernel_name(p, 2) == "void skg::scalar_kernel<2>(skg::Args)"


def test_kernel_names_exist_in_the_sources():
    """The spelled templates match the kernels' parameter lists."""
    src = open(os.path.join(bench.ROOT, "bf16_skinny_gemm_amd", "csrc", "kernels.hpp")).read()
    for sig in (r"template <int M, int LPR, int CH, int R, int KW, int XL, bool NT, int PF>\s*"
                r"__global__[^\n]*fixed_k_kernel\(Args a\)",
                r"template <int M, int U, int R, bool NT>\s*__global__[^\n]*loop_k_kernel\(Args a, int kpad\)",
                r"template <int M, int U, int R, int KW, bool NT, bool PF>\s*__global__[^\n]*mfma_kernel\(Args a\)",
                r"template <int M>\s*__global__[^\n]*scalar_kernel\(Args a\)"):
        assert re.search(sig, src), sig


def test_bytes_per_call():
    assert bench.bytes_per_call((4096, 1024, 2)) == 2 * 4096 * 1024 + 2 * 2 * 1024 + 2 * 2 * 4096
    assert bench.bytes_per_call(("pair", 4096, 128, 4)) == 4 * 4096 * 128 + 2 * 4 * 128 + 4 * 4 * 4096
    assert bench.weight_bytes((4096, 1024, 2)) == 2 * 4096 * 1024
    assert bench.weight_bytes(("pair", 4096, 128, 4)) == 4 * 4096 * 128
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_code_only_digest_ignores_notes():
    a = "int f() { return 1; } // one\n/* block\n comment */ int g;"
    b = "int f()  {\n  return 1;\n}\nint g;   // changed note"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("return 1", "return 2"))


def test_recorded_traffic(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    kern = "void skg::fixed_k_kernel<1, 64, 4, 1, 2, 0, true, 0>(skg::Args)"
    (prof / "traffic_kda.txt").write_text(
        "# a note: with a colon\nsource_digest: abc\nkernel: " + kern + "\n"
        "fetch_kib_per_dispatch: 1000\nwrite_kib_per_dispatch: 10\n"
        "copy_fetch_factor: 2.0\ncopy_write_factor: 1.0\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "abc")
    assert bench.recorded_traffic("kda", kern) == pytest.approx(1000 * 1024 * 2 + 10 * 1024)
    assert bench.recorded_traffic("kda", kern.replace("<1,", "<2,")) is None   # other kernel
    assert bench.recorded_traffic("mla", kern) is None                        # no record
    monkeypatch.setattr(bench, "source_digest", lambda: "def")
    assert bench.recorded_traffic("kda", kern) is None                        # other sources


def test_refine_same_grids_keeps_the_top_plans(tmp_path):
    import bf16_skinny_gemm_amd as skg

    recs = [_rec(1, 8, 1, 5.0, grid_blocks=0), _rec(1, 8, 1, 4.9, grid_blocks=512),
            _rec(1, 8, 1, 6.0, grid_blocks=256)]
    src = tmp_path / "s.jsonl"
    src.write_text("".join(json.dumps(r) + "\n" for r in recs))
    plans = sweep.refine_plans(skg, str(src), 1, 8, 1, False, 2, None)
    assert [p.grid_blocks for p in plans] == [512, 0]


def test_refine_twins_add_the_lookahead_form(tmp_path):
    import bf16_skinny_gemm_amd as skg

    recs = [_rec(1, 8, 2, 5.0, x_in_lds=1, grid_blocks=512),
            _rec(1, 8, 2, 5.1, rows_per_wave=2, x_in_lds=1),             # two rows: no twin
            _rec(1, 8, 2, 5.2, x_in_lds=0, prefetch=2),
            _rec(1, 8, 2, 5.3, x_in_lds=2, grid_blocks=512),             # already a twin
            _rec(1, 8, 1, 4.0, x_in_lds=1)]                              # M = 1: no twin
    src = tmp_path / "s.jsonl"
    src.write_text("".join(json.dumps(r) + "\n" for r in recs))
    plans = sweep.refine_plans(skg, str(src), 1, 8, 2, False, 4, None, twins=True)
    got = [(p.rows_per_wave, p.x_in_lds, p.prefetch, p.grid_blocks) for p in plans]
    assert got == [(1, 1, 0, 512), (1, 2, 0, 512), (2, 1, 0, 0), (1, 0, 2, 0), (1, 2, 2, 0)]
    plans = sweep.refine_plans(skg, str(src), 1, 8, 1, False, 4, None, twins=True)
    assert [(p.x_in_lds, p.grid_blocks) for p in plans] == [(1, 0)]
    plans = sweep.refine_plans(skg, str(src), 1, 8, 2, False, 1, (0, 256), twins=True)
    assert [(p.x_in_lds, p.grid_blocks) for p in plans] == [(1, 0), (2, 0), (1, 256), (2, 256)]


def test_parse_grids_refine_tokens():
    assert sweep.parse_grids("same,balanced,tile") == (sweep.SAME, sweep.BALANCED, sweep.BIG_GRID)


def test_rows_per_tile_per_kind():
    d = _rec(1, 8, 1, 1.0)["plan"]
    # fixed-K: (4 waves / k_split 2) groups x rows_per_wave 1 x 64/64 rows
    assert sweep.rows_per_tile(d) == 2
    assert sweep.rows_per_tile({**d, "lanes_per_row": 16, "rows_per_wave": 2, "k_split": 1}) == 4 * 2 * 4
    assert sweep.rows_per_tile({**d, "kind": 2, "rows_per_wave": 4, "k_split": 1}) == 16
    assert sweep.rows_per_tile({**d, "kind": 4, "rows_per_wave": 2, "k_split": 4}) == 8
    assert sweep.rows_per_tile({**d, "kind": 3}) is None


def test_balanced_grids_give_equal_tile_counts():
    # the KDA in_proj at M = 4: 256 threads, one row per wave -> 4 rows per tile, 3144 tiles
    d = _rec(12576, 4096, 4, 1.0, k_split=1, chunks=8, grid_blocks=512)["plan"]
    gs = sweep.balanced_grids(d, 12576)
    assert gs == [524, 450, 629, 393]
    tiles = 3144
    for g in gs:
        per = -(-tiles // g)
        # every block but possibly the last one takes exactly `per` tiles
        assert (g - 1) * per < tiles <= g * per
    # a pair's grid counts both weights (even blocks serve W0, odd blocks W1)
    assert sweep.balanced_grids({**d, "grid_blocks": 1024}, 12576, nmats=2) == [2 * g for g in gs]
    # the nearest to a persistent or per-tile grid are taken around 512
    assert sweep.balanced_grids({**d, "grid_blocks": 0}, 12576) == gs
    assert sweep.balanced_grids({**d, "grid_blocks": sweep.BIG_GRID}, 12576) == gs
    # nothing to balance when every block already has one tile, or for the scalar kind
    assert sweep.balanced_grids(d, 4) == []
    assert sweep.balanced_grids({**d, "kind": 3}, 12576) == []


def test_rotated_order_moves_every_plan():
    orders = [sweep.rotated_order(4, r) for r in range(3)]
    assert orders == [[0, 1, 2, 3], [1, 0, 3, 2], [2, 3, 0, 1]]
    for o in orders:
        assert sorted(o) == [0, 1, 2, 3]
    assert len({o[0] for o in orders}) == 3          # a different plan first each round
    assert sweep.rotated_order(0, 5) == []


def test_refine_same_and_balanced_grids(tmp_path):
    import bf16_skinny_gemm_amd as skg

    recs = [_rec(12576, 4096, 4, 5.0, grid_blocks=512, chunks=8, k_split=1),
            _rec(12576, 4096, 4, 5.2, grid_blocks=256, chunks=8, k_split=1),
            _rec(12576, 4096, 4, 6.0, grid_blocks=0)]
    a, b = tmp_path / "a.jsonl", tmp_path / "b.jsonl"
    a.write_text(json.dumps(recs[0]) + "\n" + json.dumps(recs[2]) + "\n")
    b.write_text(json.dumps(recs[1]) + "\n")
    plans = sweep.refine_plans(skg, f"{a},{b}", 12576, 4096, 4, False, 1,
                               (sweep.SAME, sweep.BALANCED))
    assert [p.grid_blocks for p in plans] == [512, 524, 450, 629, 393]
    assert all(p.chunks == 8 and p.k_split == 1 for p in plans)


def test_emit_inc_uses_stage_two_records_of_a_cell(tmp_path):
    fast_once = {**_rec(4096, 4096, 1, 6.0, prefetch=1), "stage": 1}
    final = [{**_rec(4096, 4096, 1, 6.5, prefetch=2), "stage": 2},
             {**_rec(4096, 4096, 1, 6.6, prefetch=0), "stage": 2}]
    other = _rec(4096, 4096, 2, 7.0, prefetch=1)                     # unstaged cell
    src = tmp_path / "s.jsonl"
    src.write_text("".join(json.dumps(r) + "\n" for r in [fast_once, *final, other]))
    out = tmp_path / "plans.inc"
    sweep.emit_inc(str(src), str(out))
    rows = re.findall(r"^\{(\d+), (\d+), (\d+), \{([^}]*)\}\},", out.read_text(), re.M)
    assert [int(v) for v in rows[0][3].split(",")][9] == 2          # not the single-pass 6.0
    assert [int(v) for v in rows[1][3].split(",")][9] == 1


def test_table_plans_reads_the_generated_table(tmp_path):
    recs = [_rec(4096, 4096, 1, 6.9, grid_blocks=1024, prefetch=2), _rec(2048, 4096, 3, 5.0)]
    src = tmp_path / "s.jsonl"
    src.write_text("".join(json.dumps(r) + "\n" for r in recs))
    out = tmp_path / "plans.inc"
    sweep.emit_inc(str(src), str(out))
    got = sweep.table_plans(str(out))
    assert got == {(2048, 4096, 3): recs[1]["plan"], (4096, 4096, 1): recs[0]["plan"]}
    # the committed table parses, one plan per (N, K, M), every field present
    committed = sweep.table_plans()
    assert len(committed) >= 100
    assert all(set(p) == set(sweep.PLAN_FIELDS) for p in committed.values())


def test_emit_inc_takes_each_cell_from_the_last_file_holding_it(tmp_path):
    first = [_rec(4096, 4096, 1, 6.0, prefetch=1), _rec(4096, 4096, 2, 7.0, prefetch=1)]
    later = [_rec(4096, 4096, 2, 7.3, prefetch=2)]                  # slower, but a later pass
    a, b = tmp_path / "a.jsonl", tmp_path / "b.jsonl"
    a.write_text("".join(json.dumps(r) + "\n" for r in first))
    b.write_text("".join(json.dumps(r) + "\n" for r in later))
    out = tmp_path / "plans.inc"
    sweep.emit_inc(f"{a},{b}", str(out))
    got = sweep.table_plans(str(out))
    assert got[(4096, 4096, 1)]["prefetch"] == 1                    # only in the first file
    assert got[(4096, 4096, 2)]["prefetch"] == 2                    # the later file decides


def test_split_trace_cuts_at_markers():
    mk = "skg::zero_kernel(void*, void*, int, int, long long, int)"
    k1 = "void skg::fixed_k_kernel<1, 64, 4, 1, 2, 0, true, 1>(skg::Args)"
    pr = "void (anonymous namespace)::read_tiles_kernel<4, true>(unsigned char const*, unsigned long long, unsigned int*)"
    rows = [(0, 5, "at::native::fill"),                     # before the first marker: ignored
            (10, 11, mk), (20, 23000, k1), (30, 33000, k1), (35, 36, mk),
            (37, 38000, k1),                                # between units (a warm-up): ignored
            (40, 41, mk), (50, 52000, pr), (55, 56, "at::native::copy"),  # torch kernels ignored
            (57, 58, mk),
            (60, 61, mk), (70, 71000, k1), (75, 76, mk)]    # wrong count: left out
    got = bench.split_trace(rows, [("a", 2), ("b", 1), ("c", 2)])
    assert got == {"a": [22.98, 32.97], "b": [51.95]}


def test_expected_trace_units_match_the_groups():
    args = bench.parse([])
    units = bench.expected_trace_units(args)
    names = [n for n, _ in units]
    assert names[:2] == ["chain:M1", "chain:M4"]
    assert dict(units)["chain:M1"] == 186 * bench.TRACE_REPLAYS["chain"]
    # every cell at M = 1, 2, 4, and a dependent chain where N >= K
    assert "cell:(77440,4096)M4" in names and "dep:(77440,4096)M4" in names
    assert "cell:(2048,4096)M1" in names and "dep:(2048,4096)M1" not in names
    assert "dep:pair2x(4096,128)M2" in names
    # copies per cell: >= 1 GiB of rotation
    assert dict(units)["cell:(4096,1024)M1"] == 128 * bench.TRACE_REPLAYS["cell"]
    assert dict(units)["cell:(77440,4096)M1"] == 2 * bench.TRACE_REPLAYS["cell"]
    assert sum(1 for n in names if n.startswith("probe:")) == 8 * len(bench.PROBE_SHAPES)
    assert [n for n in names if n.startswith("empty:")] == [f"empty:{g}" for g in bench.EMPTY_GRIDS]
    lean = bench.expected_trace_units(bench.parse(["--no-cells", "--no-probe", "--chain-ms", "1"]))
    assert lean == [("chain:M1", 186 * bench.TRACE_REPLAYS["chain"])]
    kda = bench.expected_trace_units(bench.parse(["--workload", "kda", "--no-dependent", "--no-probe"]))
    assert [n for n, _ in kda] == [f"cell:({n},4096)M{m}" for n in (12576, 4096) for m in (1, 2, 4)]


def test_chain_matches_the_decode_step():
    assert sum(n for _, _, n in bench.CHAIN) == 186 == len(bench.CHAIN_CALLS)
    assert abs(bench.chain_bytes(1) / 1e9 - 7.53) < 0.01


def test_read_kernel_trace_orders_by_start(tmp_path):
    p = tmp_path / "x_kernel_trace.csv"
    p.write_text("Kind,Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n"
                 "KERNEL_DISPATCH,2,b,200,300\nKERNEL_DISPATCH,1,a,100,150\n")
    assert bench.read_kernel_trace([str(p)]) == [(100, 150, "a"), (200, 300, "b")]


def test_dominant_kernel_pools_shapes_by_kernel_name():
    k1, k2 = "void skg::fixed_k_kernel<1, 64, 4, 1, 2, 0, true, 1>(skg::Args)", "void skg::other(skg::Args)"
    row = {"M": 1, "groups": [
        {"shape": "(12576,4096)", "calls": 34, "kernel": k1, "bytes_per_call": 100_000_000, "event_us_per_call": 10.0,
         "rocprof": {"avg_us": 11.0}},
        {"shape": "(2048,4096)", "calls": 53, "kernel": k1, "bytes_per_call": 20_000_000, "event_us_per_call": 4.0,
         "rocprof": {"avg_us": 4.5}},
        {"shape": "(4096,4096)", "calls": 34, "kernel": k2, "bytes_per_call": 50, "event_us_per_call": 6.0}]}
    r = bench.dominant_kernel(row)
    assert r["kernel"] == k1 and r["launches_per_step"] == 87
    assert r["avg_launch_us"] == pytest.approx((34 * 10 + 53 * 4) / 87, abs=1e-3)
    bpl = (34 * 100_000_000 + 53 * 20_000_000) / 87
    assert r["algorithmic_bytes_per_launch"] == round(bpl)
    assert r["achieved"] == pytest.approx(bpl / (((34 * 10 + 53 * 4) / 87) * 1e-6) / 1e9, rel=1e-4)
    assert r["rocprof_avg_launch_us"] == pytest.approx((34 * 11 + 53 * 4.5) / 87, abs=1e-3)
    assert r["share_of_step"] == pytest.approx((34 * 10 + 53 * 4) / (34 * 10 + 53 * 4 + 34 * 6), abs=1e-4)


def test_attach_read_fractions():
    cells = [{"cell": "(4096,1024)M1", "weight_bytes": 8388608, "replay_us_per_call": 3.2, "kernel_us": 3.4},
             {"cell": "(1,1)M1", "weight_bytes": 2, "replay_us_per_call": 1.0}]
    reads = [{"bytes": 8388608, "best_replay": {"replay_us": 3.0}, "best_kernel": {"kernel_us": 3.1}}]
    bench.attach_read_fractions(cells, reads)
    assert cells[0]["replay_vs_read"] == pytest.approx(3.0 / 3.2, abs=1e-4)
    assert cells[0]["kernel_vs_read"] == pytest.approx(3.1 / 3.4, abs=1e-4)
    assert "replay_vs_read" not in cells[1]


def _pmc_csv(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    head = "Dispatch_Id,Grid_Size,Workgroup_Size,Kernel_Name,Counter_Name,Counter_Value\n"
    path.write_text(head + "".join(f"{i},{g},{w},\"{k}\",{c},{v}\n" for i, (g, w, k, c, v) in enumerate(rows)))


def test_traffic_record_scales_by_the_copy(tmp_path):
    from bf16_skinny_gemm_amd import rocprof_summary as rs

    k = "void skg::fixed_k_kernel<1, 64, 4, 1, 2, 0, true, 1>(skg::Args)"
    _pmc_csv(tmp_path / "f" / "a_counter_collection.csv",
             [(1024, 256, k, "FETCH_SIZE", 100.0), (1024, 256, k, "FETCH_SIZE", 300.0),
              (64, 64, "other", "FETCH_SIZE", 9999.0)])
    _pmc_csv(tmp_path / "w" / "a_counter_collection.csv", [(1024, 256, k, "WRITE_SIZE", 2.0)])
    _pmc_csv(tmp_path / "cf" / "a_counter_collection.csv", [(8, 8, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 131072.0)])
    _pmc_csv(tmp_path / "cw" / "a_counter_collection.csv", [(8, 8, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 262144.0)])
    rec = rs.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                            k, "abc")
    d = dict(line.split(": ", 1) for line in rec.splitlines())
    assert float(d["fetch_kib_per_dispatch"]) == 200.0 and float(d["write_kib_per_dispatch"]) == 2.0
    assert float(d["copy_fetch_factor"]) == 2.0 and float(d["copy_write_factor"]) == 1.0
    assert int(d["hbm_bytes_per_dispatch"]) == 200 * 1024 * 2 + 2 * 1024
    # and bench reads the record back when the digest and kernel match
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_chain.txt").write_text("# note\n" + rec + "\n")
    import bench as b

    old_root, old_digest = b.ROOT, b.source_digest
    try:
        b.ROOT, b.source_digest = str(tmp_path), (lambda: "abc")
        assert b.recorded_traffic("chain", k) == 200 * 1024 * 2 + 2 * 1024
    finally:
        b.ROOT, b.source_digest = old_root, old_digest


def test_counter_table_derives_rates(tmp_path):
    from bf16_skinny_gemm_amd import rocprof_summary as rs

    k = "void skg::fixed_k_kernel<4, 64, 8, 1, 1, 2, true, 2>(skg::Args)"
    _pmc_csv(tmp_path / "p1" / "x_counter_collection.csv",
             [(115200, 256, k, "SQ_WAVES", 1800.0), (115200, 256, k, "VmemLatency", 2342.0),
              (115200, 256, k, "TCP_UTCL1_TRANSLATION_MISS_sum", 10.0),
              (115200, 256, k, "TCP_UTCL1_TRANSLATION_HIT_sum", 990.0),
              (115200, 256, k, "TCC_EA0_RDREQ_sum", 100.0), (115200, 256, k, "TCC_EA0_RDREQ_LEVEL_sum", 200000.0)])
    out = rs.counter_table([str(tmp_path / "p1")])
    assert "blocks=450 x 256" in out and "waves 1800" in out
    assert "vector-memory latency 2342 cycles" in out and "(1.00% miss)" in out
    assert "L2->DRAM read latency 2000 cycles" in out


def test_bench_tables_render_a_line():
    from bf16_skinny_gemm_amd import rocprof_summary as rs

    line = {"chains": [{"M": 1, "ms_per_step": 1.4, "calls": 186, "gbps": 5400.0, "frac_of_peak": 0.675,
                        "parity": {"pass": True, "outputs_checked": 186, "elements": 10, "max_g1_ratio": 0.1,
                                   "max_s1_ratio": 0.9, "min_row_cosine": 0.99999999},
                        "groups": [{"shape": "(4096,4096)", "calls": 34, "kernel": "void skg::k(skg::Args)",
                                    "event_us_per_call": 6.7, "event_frac": 0.626}]}],
            "cells": [{"cell": "(4096,4096)M1", "replay_us_per_call": 6.69, "replay_frac": 0.627,
                       "read_probe_replay_us": 6.55, "rocprof": {"avg_us": 7.0, "med_us": 6.9}, "kernel_frac": 0.6,
                       "cpu_oracle_us": 2876.0, "parity": {"pass": True}}],
            "read_probe": [{"bytes": 8, "best_replay": {"loads": 4, "threads": 256, "replay_us": 1.0},
                            "replay_gbps": 0.01, "all": [{"loads": 4, "threads": 256, "replay_us": 1.0}]}],
            "empty_kernel": [{"grid": 1, "replay_us_per_launch": 1.56}]}
    out = rs.bench_tables(line)
    assert "1400.0 µs per step of 186 calls" in out and "| (4096,4096) | 34 | `k(skg::Args)` | 6.700 | 62.6 |" in out
    assert "| (4096,4096)M1 | 7.000 (6.900) | 60.0 | 6.690 | 62.7 |" in out
    assert "| 1 | 1.56 | n/a |" in out


def test_split_k_report(tmp_path):
    """Table plan vs fastest split-K plan per cell, from the round records when present."""
    from bf16_skinny_gemm_amd import sweep

    def rec(M, kind, us, stage=None, S=0):
        plan = {"kind": kind, "threads_per_block": 256, "lanes_per_row": 64, "chunks": 2,
                "rows_per_wave": 1, "k_split": S, "nontemporal": 1, "grid_blocks": 0,
                "x_in_lds": 0, "prefetch": 0}
        r = {"N": 2048, "K": 4096, "M": M, "pair": False, "plan": plan, "us": us}
        if stage:
            r["stage"] = stage
        return json.dumps(r)

    lines = [rec(1, 1, 4.4, 1), rec(1, 5, 5.0, 1, S=4), rec(1, 5, 3.0, 1, S=8),  # single pass
             rec(1, 1, 4.5, 2), rec(1, 5, 5.9, 2, S=4),                        # rounds decide
             rec(2, 1, 4.7), rec(2, 5, 6.0, S=2),
             json.dumps({"N": 2048, "K": 4096, "M": 2, "pair": False, "complete": True})]
    p = tmp_path / "s.jsonl"
    p.write_text("\n".join(lines) + "\n")
    out = sweep.split_k_report(str(p)).splitlines()
    assert out[2] == "| (2048,4096) | 1 | 4.500 | 5.900 | 1.31 | (64, 2, 1, 4, 256) |"
    assert out[3] == "| (2048,4096) | 2 | 4.700 | 6.000 | 1.28 | (64, 2, 1, 2, 256) |"
    assert len(out) == 4


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says so,
    before touching any device."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=root)
    assert res.returncode == 2, res.stderr
    assert "one GPU" in res.stderr and res.stdout == ""
