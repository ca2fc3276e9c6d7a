"""C-ABI contract of libskinny_gemm_bf16.so, checked without running any kernel.

Argument validation happens before the library touches a device, so the
error paths are exercised here on the CPU with fake (never dereferenced)
pointers.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


@pytest.fixture(scope="module")
def skg():
    from bf16_skinny_gemm_amd.build import LIB_PATH

    if not os.path.exists(LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    import bf16_skinny_gemm_amd

    bf16_skinny_gemm_amd.lib()
    return bf16_skinny_gemm_amd


PROBE_HEADER = "skinny_stream_probe.h"


def declared_functions(headers=None):
    """Functions declared in include/*.h (or in the named headers only)."""
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if not fn.endswith(".h") or (headers is not None and fn not in headers):
            continue
        text = open(os.path.join(HEADER_DIR, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(skinny_\w+)\s*\(", text, flags=re.M):
            names.append(m.group(1))
    return names


def gemm_headers():
    return [f for f in os.listdir(HEADER_DIR) if f.endswith(".h") and f != PROBE_HEADER]


def test_header_declares_entry_points():
    names = declared_functions()
    for want in ("skinny_gemm_bf16", "skinny_gemm_bf16_pair", "skinny_gemm_bf16_ex",
                 "skinny_gemm_bf16_pair_ex", "skinny_gemm_init", "skinny_gemm_get_plan",
                 "skinny_gemm_num_variants", "skinny_gemm_get_variant",
                 "skinny_gemm_status_string", "skinny_gemm_version"):
        assert want in names


def test_library_exports_every_declared_symbol(skg):
    L = skg.lib()
    for name in declared_functions(gemm_headers()):
        assert hasattr(L, name), f"{name} declared in include/ but not exported"


def test_probe_library_exports_and_validates(skg):
    """The read-stream probe's library exports what its header declares and refuses
    bad arguments before touching a device."""
    from bf16_skinny_gemm_amd import probe

    L = probe.lib()
    names = declared_functions([PROBE_HEADER])
    assert names == ["skinny_probe_sink_words", "skinny_probe_read", "skinny_probe_tiles_sink_words",
                     "skinny_probe_read_tiles", "skinny_probe_empty"]
    for name in names:
        assert hasattr(L, name)
    assert probe.sink_words(3) == 3 * 256 and probe.sink_words(0) == 0
    buf, sink = 0x10000000, 0x20000000  # never dereferenced: every call below is refused
    for args in ((buf, 100, 1, 8, sink),        # bytes not a multiple of 16
                 (buf, 4096, 1, 0, sink),       # no blocks
                 (buf, 4096, 1, 65537, sink),   # too many blocks
                 (buf, 4096, 1, 8, None),       # no sink
                 (None, 4096, 1, 8, sink),      # no buffer
                 (buf + 8, 4096, 1, 8, sink),   # misaligned buffer
                 (buf, 4096, 1, 8, buf + 64)):  # sink inside the buffer
        assert L.skinny_probe_read(*args, None) == -1, args
    # the one-block-per-tile reader: one sink word per wave, refused shapes give 0 words
    assert probe.tiles_sink_words(1 << 20, 4, 256) == (1 << 20) // (16 << 10) * 4
    assert probe.tiles_sink_words((1 << 20) + 16, 4, 256) == ((1 << 20) // (16 << 10) + 1) * 4
    assert probe.tiles_sink_words(4096, 3, 256) == 0 and probe.tiles_sink_words(4096, 4, 96) == 0
    for args in ((buf, 100, 1, 4, 256, sink),        # bytes not a multiple of 16
                 (buf, 0, 1, 4, 256, sink),          # nothing to read
                 (buf, 4096, 1, 5, 256, sink),       # loads not 2, 4, 8 or 16
                 (buf, 4096, 1, 4, 100, sink),       # threads not a multiple of 64
                 (buf, 4096, 1, 4, 2048, sink),      # too many threads
                 (buf, 4096, 1, 4, 256, None),       # no sink
                 (None, 4096, 1, 4, 256, sink),      # no buffer
                 (buf + 8, 4096, 1, 4, 256, sink),   # misaligned buffer
                 (buf, 4096, 1, 4, 256, buf + 64)):  # sink inside the buffer
        assert L.skinny_probe_read_tiles(*args, None) == -1, args
    for grid, threads in ((0, 256), (1 << 25, 256), (8, 32), (8, 2048), (8, 100)):
        assert L.skinny_probe_empty(grid, threads, None) == -1, (grid, threads)


def test_exports_have_c_linkage(skg):
    from bf16_skinny_gemm_amd.build import LIB_PATH

    # C symbols are plain names in the dynamic symbol table (no C++ mangling)
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions(gemm_headers()):
        assert name in syms


def test_status_strings(skg):
    for st, tag in ((0, "SKINNY_OK"), (-1, "INVALID_ARG"), (-2, "UNSUPPORTED"),
                    (-3, "NOT_INITIALIZED"), (-4, "LAUNCH"), (12345, "UNKNOWN")):
        assert tag in skg.skinny_gemm_status_string(st)


def test_version(skg):
    assert skg.skinny_gemm_version() >= 100


def test_variants_enumerate(skg):
    n = skg.skinny_gemm_num_variants()
    assert n > 10
    kinds = set()
    for i in range(n):
        p = skg.skinny_gemm_get_variant(i)
        kinds.add(p.kind)
        assert p.threads_per_block % 64 == 0 and p.grid_blocks == 0
        assert p.lanes_per_row in (8, 16, 32, 64)
        assert p.k_split in (1, 2, 4, 8)
    assert kinds == {1, 2, 3, 4}
    with pytest.raises(skg.SkinnyError):
        skg.skinny_gemm_get_variant(n)
    with pytest.raises(skg.SkinnyError):
        skg.skinny_gemm_get_variant(-1)


def _fixed_k(p):
    return p.k_split * p.lanes_per_row * 8 * p.chunks


def test_default_plans(skg):
    # every decode projection shape has a vector plan at every M (tuned or default);
    # the 4x4x4 MFMA family has 4 rows of A, so never beyond M = 4
    for (N, K) in [(4096, 1024), (12576, 4096), (4096, 4096), (2048, 4096), (8192, 1536),
                   (4096, 8192), (77440, 4096), (4096, 128)]:
        for M in range(1, 9):
            p, _ = skg.skinny_gemm_get_plan(N, K, M)
            assert p.kind in (skg.SKINNY_KIND_FIXED_K, skg.SKINNY_KIND_LOOP_K,
                              skg.SKINNY_KIND_MFMA), (N, K, M, p)
            assert M <= 4 or p.kind != skg.SKINNY_KIND_MFMA, (N, K, M, p)
            if p.kind == skg.SKINNY_KIND_FIXED_K:
                assert _fixed_k(p) == K
            if p.kind == skg.SKINNY_KIND_MFMA:
                assert K % (128 * p.k_split) == 0 and (K // (128 * p.k_split)) % p.chunks == 0
    # an unlisted K that a compile-time-K variant covers gets that variant by default
    p, tuned = skg.skinny_gemm_get_plan(1000, 4096, 1)
    assert not tuned and p.kind == skg.SKINNY_KIND_FIXED_K and _fixed_k(p) == 4096
    p, tuned = skg.skinny_gemm_get_plan(100, 1000, 2)
    assert p.kind == skg.SKINNY_KIND_LOOP_K and not tuned
    p, _ = skg.skinny_gemm_get_plan(100, 1001, 2)
    assert p.kind == skg.SKINNY_KIND_SCALAR


def test_plan_table_entries_are_valid(skg):
    """Every tuned entry names a compiled variant compatible with its K."""
    inc = os.path.join(ROOT, "bf16_skinny_gemm_amd", "csrc", "plans_gfx950.inc")
    rows = re.findall(r"^\s*\{\s*(\d+),\s*(\d+),\s*(\d+),\s*\{([^}]*)\}\s*\},", open(inc).read(), re.M)
    keys = set()
    vset = {tuple(v.as_dict()[k] for k in ("kind", "lanes_per_row", "chunks", "rows_per_wave",
                                           "k_split", "nontemporal", "x_in_lds", "prefetch"))
            for v in skg.variants()}
    for N, K, M, fields in rows:
        N, K, M = int(N), int(K), int(M)
        assert (N, K, M) not in keys, f"duplicate plan key {(N, K, M)}"
        keys.add((N, K, M))
        p, tuned = skg.skinny_gemm_get_plan(N, K, M)
        assert tuned
        vals = [int(v) for v in fields.split(",")]
        assert vals == [p.kind, p.threads_per_block, p.lanes_per_row, p.chunks, p.rows_per_wave,
                        p.k_split, p.nontemporal, p.grid_blocks, p.x_in_lds, p.prefetch]
        assert (p.kind, p.lanes_per_row, p.chunks, p.rows_per_wave, p.k_split, p.nontemporal,
                p.x_in_lds, p.prefetch) in vset
        if p.kind == skg.SKINNY_KIND_FIXED_K:
            assert _fixed_k(p) == K
        if p.kind == skg.SKINNY_KIND_MFMA:
            assert K % (128 * p.k_split) == 0 and (K // (128 * p.k_split)) % p.chunks == 0
        assert 1 <= M <= 8 and p.threads_per_block // 64 % p.k_split == 0
        assert M <= 4 or p.kind != skg.SKINNY_KIND_MFMA


def test_get_plan_rejects(skg):
    for args in ((0, 128, 1), (128, 0, 1), (128, 128, 0), (128, 128, 9)):
        with pytest.raises(skg.SkinnyError):
            skg.skinny_gemm_get_plan(*args)
    L = skg.lib()
    assert L.skinny_gemm_get_plan(128, 128, 1, None) == skg.SKINNY_ERR_INVALID_ARG


# --- validation before any device work (fake addresses, never dereferenced) ---

X = 0x7F0000000000
W = 0x7F0000100000
Y = 0x7F0000900000
W1 = 0x7F0001000000
Y1 = 0x7F0002000000


def _call(L, *a):
    return L.skinny_gemm_bf16(*a)


@pytest.mark.parametrize("args", [
    (X, W, Y, 9, 16, 16, None),          # M > 8
    (X, W, Y, -1, 16, 16, None),         # negative M
    (X, W, Y, 1, -3, 16, None),          # negative N
    (X, W, Y, 1, 16, -8, None),          # negative K
    (None, W, Y, 1, 16, 16, None),       # null x
    (X, None, Y, 1, 16, 16, None),       # null W
    (X, W, None, 1, 16, 16, None),       # null y
    (X + 1, W, Y, 1, 16, 16, None),      # odd address
    (X, W, X + 8, 1, 16, 16, None),      # y overlaps x
    (X, W, W + 64, 2, 16, 16, None),     # y overlaps W
])
def test_single_invalid_args(skg, args):
    assert _call(skg.lib(), *args) == skg.SKINNY_ERR_INVALID_ARG


def test_pair_invalid_args(skg):
    L = skg.lib()
    ok = (X, W, W1, Y, Y1, 1, 16, 16, None)
    bad = [
        (X, W, None, Y, Y1, 1, 16, 16, None),   # null W1
        (X, W, W1, Y, None, 1, 16, 16, None),   # null y1
        (X, W, W1, Y, Y + 16, 1, 16, 16, None),  # y0 and y1 overlap
        (X, W, W1, Y, W1 + 32, 1, 16, 16, None),  # y1 overlaps W1
        (X, W, W1, Y, Y1, 9, 16, 16, None),     # M out of range
    ]
    for b in bad:
        assert L.skinny_gemm_bf16_pair(*b) == skg.SKINNY_ERR_INVALID_ARG, b
    assert ok  # the valid form needs a device; it is exercised by the GPU tests


def test_empty_calls_are_noops(skg):
    L = skg.lib()
    # M == 0 or N == 0: nothing to do, any pointers (even NULL) accepted, no device needed
    assert L.skinny_gemm_bf16(None, None, None, 0, 16, 16, None) == skg.SKINNY_OK
    assert L.skinny_gemm_bf16(None, None, None, 2, 0, 16, None) == skg.SKINNY_OK
    assert L.skinny_gemm_bf16_pair(None, None, None, None, None, 0, 4, 4, None) == skg.SKINNY_OK


def test_ex_rejects_bad_plans(skg):
    L = skg.lib()
    Plan = skg.Plan
    assert L.skinny_gemm_bf16_ex(X, W, Y, 1, 16, 1024, None, None) == skg.SKINNY_ERR_INVALID_ARG
    # a plan that names no compiled variant
    p = Plan(kind=1, threads_per_block=256, lanes_per_row=64, chunks=7, rows_per_wave=1,
             k_split=1, nontemporal=0, grid_blocks=0)
    assert L.skinny_gemm_bf16_ex(X, W, Y, 1, 16, 1024, ctypes.byref(p), None) == \
        skg.SKINNY_ERR_UNSUPPORTED
    # compiled variant, wrong K for a fixed-K plan
    p = Plan(kind=1, threads_per_block=256, lanes_per_row=64, chunks=2, rows_per_wave=1,
             k_split=1, nontemporal=1, grid_blocks=0, prefetch=1)
    assert L.skinny_gemm_bf16_ex(X, W, Y, 1, 16, 2048, ctypes.byref(p), None) == \
        skg.SKINNY_ERR_INVALID_ARG
    # x_in_lds: 0, 1 or 2 for a fixed-K plan, 1 for looped-K
    p = Plan(kind=1, threads_per_block=256, lanes_per_row=64, chunks=2, rows_per_wave=1,
             k_split=1, nontemporal=1, grid_blocks=0, x_in_lds=3, prefetch=1)
    assert L.skinny_gemm_bf16_ex(X, W, Y, 2, 16, 1024, ctypes.byref(p), None) in \
        (skg.SKINNY_ERR_INVALID_ARG, skg.SKINNY_ERR_UNSUPPORTED)
    p = Plan(kind=2, threads_per_block=256, lanes_per_row=64, chunks=4, rows_per_wave=1,
             k_split=1, nontemporal=1, grid_blocks=0, x_in_lds=2)
    assert L.skinny_gemm_bf16_ex(X, W, Y, 2, 16, 1024, ctypes.byref(p), None) in \
        (skg.SKINNY_ERR_INVALID_ARG, skg.SKINNY_ERR_UNSUPPORTED)
    # x read one chunk ahead is compiled for M >= 2 only
    p = Plan(kind=1, threads_per_block=256, lanes_per_row=64, chunks=2, rows_per_wave=1,
             k_split=1, nontemporal=1, grid_blocks=0, x_in_lds=2, prefetch=1)
    assert L.skinny_gemm_bf16_ex(X, W, Y, 1, 16, 1024, ctypes.byref(p), None) == \
        skg.SKINNY_ERR_UNSUPPORTED
    # block size not a multiple of 64 * k_split, too large, negative grid
    for tpb, ks, ch, grid in ((96, 1, 2, 0), (1024, 1, 2, 0), (64, 2, 1, 0), (256, 1, 2, -1)):
        p = Plan(kind=1, threads_per_block=tpb, lanes_per_row=64, chunks=ch, rows_per_wave=1,
                 k_split=ks, nontemporal=1, grid_blocks=grid, prefetch=1)
        assert L.skinny_gemm_bf16_ex(X, W, Y, 1, 16, 1024, ctypes.byref(p), None) == \
            skg.SKINNY_ERR_INVALID_ARG, (tpb, ks, grid)
    # a vector plan on a misaligned pointer or K % 8 != 0 is an error, not a silent fallback
    p = Plan(kind=2, threads_per_block=256, lanes_per_row=64, chunks=4, rows_per_wave=1,
             k_split=1, nontemporal=0, grid_blocks=0, x_in_lds=1)
    assert L.skinny_gemm_bf16_ex(X + 2, W, Y, 1, 16, 1000, ctypes.byref(p), None) == \
        skg.SKINNY_ERR_INVALID_ARG


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-device path")
def test_no_device(skg):
    L = skg.lib()
    # with no GPU present, a valid call cannot run and says so instead of crashing
    st = L.skinny_gemm_bf16(X, W, Y, 1, 16, 16, None)
    assert st in (skg.SKINNY_ERR_UNSUPPORTED, skg.SKINNY_ERR_INVALID_ARG)
    assert L.skinny_gemm_init(0) in (skg.SKINNY_ERR_UNSUPPORTED, skg.SKINNY_ERR_INVALID_ARG)
    assert L.skinny_gemm_init(-1) == skg.SKINNY_ERR_INVALID_ARG


def test_pair_strided_validation(skg):
    """Strides below the row length and outputs that share elements are rejected
    before any device work; outputs interleaved in one merged tensor are valid (on a
    machine without a GPU such a call gets past validation and stops at the device
    check)."""
    L = skg.lib()
    M, N, K = 2, 16, 32
    x0, x1 = X, X + 2 * K
    y0 = Y
    bad = [
        (x0, x1, K - 1, W, W1, y0, Y1, N, M, N, K),          # ldx < K
        (x0, x1, 2 * K, W, W1, y0, Y1, N - 1, M, N, K),      # ldy < N
        (x0, x1, 2 * K, W, W1, y0, y0 + 2, 2 * N, M, N, K),  # y1 overlaps y0's rows
        (x0, x1, 2 * K, W, W1, y0, x1 + 4, N, M, N, K),      # y1 overlaps x1
        (x0, None, 2 * K, W, W1, y0, Y1, N, M, N, K),        # null x1
    ]
    for b in bad:
        assert L.skinny_gemm_bf16_pair_strided(*b, None) == skg.SKINNY_ERR_INVALID_ARG, b
    # merged output [M][2N]: y1 = y0 + N elements, ldy = 2N -> disjoint, accepted
    ok = (x0, x1, 2 * K, W, W1, y0, y0 + 2 * N, 2 * N, M, N, K)
    if not __import__("torch").cuda.is_available():
        assert L.skinny_gemm_bf16_pair_strided(*ok, None) == skg.SKINNY_ERR_UNSUPPORTED


def test_plan_table_covers_the_decode_shapes():
    """The generated table holds rows for M = 1..8 of every decode shape (the
    configurations' shapes, the paired (4096,128) and (2048,128), the router gate,
    the merged f_a/g_a and the TP4/TP8 rank shapes); the GPU parity suite runs
    each of them at full size."""
    path = os.path.join(ROOT, "bf16_skinny_gemm_amd", "csrc", "plans_gfx950.inc")
    cells = {}
    for n, k, m in re.findall(r"^\{(\d+), (\d+), (\d+), \{", open(path).read(), re.M):
        cells.setdefault((int(n), int(k)), set()).add(int(m))
    want = [(4096, 1024), (12576, 4096), (4096, 4096), (2048, 4096), (8192, 1536), (4096, 8192),
            (77440, 4096), (4096, 128), (2048, 128), (288, 4096), (256, 4096), (6416, 4096),
            (19360, 4096), (38720, 4096)]
    assert sorted(cells) == sorted(want)
    for s in want:
        assert cells[s] == set(range(1, 9)), s


# ---------------------------------------------------------------------------
# cross-block split-K: host-side contract (sizes, plans, refusals)
# ---------------------------------------------------------------------------

def _split_plan(skg, lanes=64, chunks=2, rows=1, S=4, tpb=256, **kw):
    d = dict(kind=skg.SKINNY_KIND_SPLIT_K, threads_per_block=tpb, lanes_per_row=lanes, chunks=chunks,
             rows_per_wave=rows, k_split=S, nontemporal=1, grid_blocks=0, x_in_lds=0, prefetch=0)
    d.update(kw)
    return skg.Plan(**d)


def test_split_k_variants_and_defaults(skg):
    vs = skg.split_k_variants()
    assert len(vs) == skg.skinny_gemm_split_k_num_variants() > 0
    for v in vs:
        assert v.kind == skg.SKINNY_KIND_SPLIT_K and v.k_split == 0 and v.grid_blocks == 0
    with pytest.raises(skg.SkinnyError):
        skg.skinny_gemm_split_k_get_variant(len(vs))
    # the default: 256 threads, one row per wave, S tried in 4, 2, 8 order
    for K, lanes, chunks, S in ((4096, 64, 2, 4), (8192, 64, 4, 4), (1024, 64, 1, 2),
                                (2048, 64, 1, 4), (1536, 32, 3, 2)):
        p = skg.skinny_gemm_split_k_default_plan(1, 4096, K)
        assert (p.lanes_per_row, p.chunks, p.rows_per_wave, p.k_split, p.threads_per_block) == \
            (lanes, chunks, 1, S, 256), K
        assert S * lanes * 8 * chunks == K
    for K in (1000, 12288, 8):
        with pytest.raises(skg.SkinnyError) as e:
            skg.skinny_gemm_split_k_default_plan(1, 4096, K)
        assert e.value.status == skg.SKINNY_ERR_UNSUPPORTED


def test_split_k_workspace_bytes(skg):
    """64 KiB of tile counters, then S*M*N float partials."""
    for M, N, K, tpb, rows, lanes, chunks, S in ((1, 4096, 4096, 256, 1, 64, 2, 4),
                                                 (4, 1000, 4096, 256, 2, 64, 4, 2),
                                                 (8, 77, 1536, 64, 1, 32, 3, 2)):
        p = _split_plan(skg, lanes, chunks, rows, S, tpb)
        assert skg.skinny_gemm_split_k_workspace_bytes(M, N, K, p) == 65536 + S * M * N * 4
    # 16384 tiles at most: 4 rows per tile at 256 threads, one row per wave
    assert skg.skinny_gemm_split_k_workspace_bytes(1, 4 * 16384, 4096, _split_plan(skg)) > 0
    assert skg.skinny_gemm_split_k_workspace_bytes(1, 4 * 16384 + 1, 4096, _split_plan(skg)) == 0
    # refused: M out of range, K not S * slice, bad plan fields
    assert skg.skinny_gemm_split_k_workspace_bytes(9, 4096, 4096, None) == 0
    assert skg.skinny_gemm_split_k_workspace_bytes(0, 4096, 4096, None) == 0
    assert skg.skinny_gemm_split_k_workspace_bytes(1, 4096, 2048, _split_plan(skg)) == 0
    for bad in (dict(grid_blocks=4), dict(x_in_lds=1), dict(prefetch=1), dict(nontemporal=0),
                dict(tpb=96), dict(tpb=1024), dict(S=0), dict(kind=1), dict(chunks=5)):
        kw = dict(bad)
        tpb = kw.pop("tpb", 256)
        S = kw.pop("S", 4)
        assert skg.skinny_gemm_split_k_workspace_bytes(1, 4096, 4096, _split_plan(skg, S=S, tpb=tpb, **kw)) == 0, bad


def test_split_k_refusals_need_no_device(skg):
    """Every refusal below is decided before the library looks for a device."""
    L = skg.lib()
    x, W, y, ws = 0x10000000, 0x20000000, 0x30000000, 0x40000000  # never dereferenced
    M, N, K = 2, 1024, 4096
    p = _split_plan(skg)
    need = skg.skinny_gemm_split_k_workspace_bytes(M, N, K, p)
    E = skg.SKINNY_ERR_INVALID_ARG
    call = L.skinny_gemm_bf16_split_k
    r = ctypes.byref
    assert call(x, W, y, M, N, K, r(p), ws, need - 1, None) == E      # workspace too small
    assert call(x, W, y, M, N, K, r(p), None, need, None) == E        # no workspace
    assert call(x, W, y, M, N, K, r(p), ws + 128, need, None) == E    # not 256-byte aligned
    assert call(x, W, y, M, N, K, r(p), y, need, None) == E           # workspace over y
    assert call(x, W, y, M, N, K, r(p), W - 256, need, None) == E     # workspace over W
    assert call(x, W, y, M, N, 2048, r(p), ws, need, None) == E       # K != S * slice
    assert call(x + 8, W, y, M, N, K, r(p), ws, need, None) == E      # x not 16-byte aligned
    assert call(x, W, y, M, N, K - 4, None, ws, need, None) == E      # K % 8 != 0
    assert call(x, W, y, 9, N, K, None, ws, need, None) == E          # M > 8
    assert call(x, W, y, M, N, 0, None, ws, need, None) == E          # K == 0
    assert call(x, W, None, M, N, K, r(p), ws, need, None) == E       # no y
    assert call(x, W, x, M, N, K, r(p), ws, need, None) == E          # y over x
    # nothing to do: M == 0 or N == 0 is a no-op with any pointers
    assert call(None, None, None, 0, N, K, None, None, 0, None) == skg.SKINNY_OK
    assert call(None, None, None, M, 0, K, None, None, 0, None) == skg.SKINNY_OK


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-device path")
def test_split_k_no_device(skg):
    L = skg.lib()
    p = _split_plan(skg)
    need = skg.skinny_gemm_split_k_workspace_bytes(2, 1024, 4096, p)
    st = L.skinny_gemm_bf16_split_k(0x10000000, 0x20000000, 0x30000000, 2, 1024, 4096, ctypes.byref(p),
                                    0x40000000, need, None)
    assert st in (skg.SKINNY_ERR_UNSUPPORTED, skg.SKINNY_ERR_INVALID_ARG)


def test_split_k_noalloc_refusals_need_no_device(skg):
    """The static workspace's limits are checked before any device work."""
    L = skg.lib()
    x, W, y = 0x10000000, 0x40000000, 0x80000000  # never dereferenced
    p = _split_plan(skg)  # S = 4 at K = 4096, 4 rows per tile
    E = skg.SKINNY_ERR_INVALID_ARG
    call = L.skinny_gemm_bf16_split_k_noalloc
    assert call(x, W, y, 8, 32769, 4096, ctypes.byref(p), None) == E  # S*M*N > 2^20
    assert call(x, W, y, 1, 4 * 16384 + 4, 4096, ctypes.byref(p), None) == E  # > 16384 tiles
    assert call(x, W, y, 9, 1024, 4096, None, None) == E
    assert call(x + 8, W, y, 1, 1024, 4096, None, None) == E
    assert call(x, W, None, 1, 1024, 4096, None, None) == E
    assert call(None, None, None, 0, 1024, 4096, None, None) == skg.SKINNY_OK


def test_default_plan_takes_nearest_tuned_neighbour(skg):
    """A shape the table does not hold takes the tuned plan of the nearest N (by
    ratio) with the same K and M, a tuned block count turned into the persistent
    grid (0); a K the table never tuned takes looped-K, with 512 threads per block
    once the staged x (M*K*2 bytes) reaches 32 KiB."""
    import math

    inc = os.path.join(ROOT, "bf16_skinny_gemm_amd", "csrc", "plans_gfx950.inc")
    fields = ("kind", "threads_per_block", "lanes_per_row", "chunks", "rows_per_wave", "k_split",
              "nontemporal", "grid_blocks", "x_in_lds", "prefetch")
    table = {}
    for n, k, m, f in re.findall(r"^\s*\{\s*(\d+),\s*(\d+),\s*(\d+),\s*\{([^}]*)\}\s*\},", open(inc).read(), re.M):
        table[(int(n), int(k), int(m))] = dict(zip(fields, (int(v) for v in f.split(","))))
    checked = 0
    for N in (300, 1000, 3000, 6144, 9000, 14336, 30000, 100000):
        for K in (1024, 1536, 4096, 8192):
            for M in range(1, 9):
                near = [(abs(math.log(n / N)), n) for (n, k, m) in table if k == K and m == M]
                if not near or (N, K, M) in table:
                    continue
                want = dict(table[(min(near)[1], K, M)])
                if 0 < want["grid_blocks"] < (1 << 20):
                    want["grid_blocks"] = 0
                p, tuned = skg.skinny_gemm_get_plan(N, K, M)
                assert not tuned and p.as_dict() == want, (N, K, M, p, want)
                checked += 1
    assert checked > 100
    for N, K, M, tpb in ((4096, 14336, 1, 256), (4096, 14336, 4, 512), (2048, 2048, 4, 256),
                         (5120, 5120, 4, 512), (100, 1000, 2, 256)):
        p, tuned = skg.skinny_gemm_get_plan(N, K, M)
        assert not tuned and p.kind == skg.SKINNY_KIND_LOOP_K and p.threads_per_block == tpb, (N, K, M, p)
