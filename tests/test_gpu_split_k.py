"""Cross-block split-K (skinny_gemm_bf16_split_k) against the CPU oracle on an
MI355X (gfx950), through the C ABI.

The bar is the parity suite's (oracle/accept.py: G1 per element, G2 per output
row, S1). Beyond it, split-K must give the same bits as the in-block FIXED_K plan
with the same (lanes_per_row, chunks, k_split): both add each slice's chunks in
the same order, meet the lanes by the same butterfly and add the slices 0..S-1.
Its arrival counters must be back at zero after every call, which the repeated
calls, the shape changes on one workspace and the graph replays check: a counter
left non-zero would leave some tile with no last block, and its outputs unwritten.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

# the decode projections whose K splits over blocks (N, K), at full size
DECODE = [(2048, 4096), (4096, 8192), (4096, 4096), (4096, 1024), (8192, 1536), (12576, 4096)]


@pytest.fixture(scope="module")
def skg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bf16_skinny_gemm_amd as m

    m.skinny_gemm_init(torch.cuda.current_device())
    return m


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check(y_dev, x, W, label=""):
    yr, ref, mag = oracle.gemm(x, W)
    res = oracle.acceptance(to_host(y_dev), yr, ref, mag)
    assert res["pass"], f"{label}: {res}"
    return res


def split_plan(skg, lanes, chunks, rows, S, tpb=256):
    return skg.Plan(kind=skg.SKINNY_KIND_SPLIT_K, threads_per_block=tpb, lanes_per_row=lanes,
                    chunks=chunks, rows_per_wave=rows, k_split=S, nontemporal=1, grid_blocks=0,
                    x_in_lds=0, prefetch=0)


def fixed_plan(skg, lanes, chunks, rows, S, tpb=256):
    return skg.Plan(kind=skg.SKINNY_KIND_FIXED_K, threads_per_block=tpb, lanes_per_row=lanes,
                    chunks=chunks, rows_per_wave=rows, k_split=S, nontemporal=1, grid_blocks=0,
                    x_in_lds=0, prefetch=0)


def nan_fill(t: torch.Tensor) -> None:
    t.view(torch.int16).fill_(0x7FC0)


# ---------------------------------------------------------------------------
# every split-K variant, every M, S = 1..16, several tiles and a ragged tail
# ---------------------------------------------------------------------------

def _variants():
    import bf16_skinny_gemm_amd as m

    try:
        return [pytest.param(v, id=f"l{v.lanes_per_row}-c{v.chunks}-r{v.rows_per_wave}")
                for v in m.split_k_variants()]
    except Exception:
        return [pytest.param(None, id="no-library")]


@pytest.mark.parametrize("variant", _variants())
def test_every_split_variant(skg, variant):
    assert variant is not None, "library missing"
    ran = 0
    for S in (1, 2, 4, 8, 16):
        K = S * variant.lanes_per_row * 8 * variant.chunks
        for tpb in (256, 64):
            rows_t = tpb // 64 * variant.rows_per_wave * (64 // variant.lanes_per_row)
            N = 3 * rows_t + 5  # four tiles, the last one ragged
            W = synth.weights(N, K, seed=3, shape_id=K, tensor_id=S)
            Wd = to_dev(W)
            for M in range(1, 9):
                plan = split_plan(skg, variant.lanes_per_row, variant.chunks, variant.rows_per_wave, S, tpb)
                nbytes = skg.skinny_gemm_split_k_workspace_bytes(M, N, K, plan)
                if nbytes == 0:  # this M is beyond the variant's register budget
                    continue
                x = synth.activations(M, K, seed=3, shape_id=K, tensor_id=100 + M)
                xd = to_dev(x)
                ws = skg.split_k_workspace(M, N, K, plan)
                y = skg.gemm_split_k(xd, Wd, ws, plan=plan)
                check(y, x, W, f"S={S} tpb={tpb} M={M} N={N} K={K}")
                ran += 1
    assert ran > 0


# ---------------------------------------------------------------------------
# the same bits as the in-block plan with the same (lanes, chunks, k_split)
# ---------------------------------------------------------------------------

BITWISE = [  # (K, lanes, chunks, rows, S)
    (4096, 64, 2, 1, 4), (4096, 64, 2, 2, 4), (4096, 64, 4, 1, 2), (4096, 64, 4, 2, 2),
    (4096, 64, 8, 1, 1), (8192, 64, 4, 1, 4), (8192, 64, 4, 2, 4), (8192, 64, 8, 1, 2),
    (1024, 64, 1, 1, 2), (1024, 64, 1, 2, 2), (1024, 64, 2, 1, 1), (1536, 32, 3, 1, 2),
]


@pytest.mark.parametrize("K,lanes,chunks,rows,S", BITWISE)
def test_split_equals_in_block(skg, K, lanes, chunks, rows, S):
    N = 1000
    W = synth.weights(N, K, seed=4, shape_id=K, tensor_id=lanes * 100 + chunks)
    Wd = to_dev(W)
    compared = 0
    for M in range(1, 9):
        sp = split_plan(skg, lanes, chunks, rows, S)
        if skg.skinny_gemm_split_k_workspace_bytes(M, N, K, sp) == 0:
            continue
        xd = to_dev(synth.activations(M, K, seed=4, shape_id=K, tensor_id=M))
        try:
            yf = skg.gemm(xd, Wd, plan=fixed_plan(skg, lanes, chunks, rows, S))
        except skg.SkinnyError as e:
            assert e.status == skg.SKINNY_ERR_UNSUPPORTED  # the in-block instance is not built at this M
            continue
        ys = skg.gemm_split_k(xd, Wd, skg.split_k_workspace(M, N, K, sp), plan=sp)
        assert np.array_equal(to_host(ys), to_host(yf)), f"M={M}"
        compared += 1
    assert compared > 0


# ---------------------------------------------------------------------------
# decode shapes at full size, default plan, M = 1..8
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", DECODE)
def test_decode_shapes_full(skg, N, K):
    W = synth.weights(N, K, seed=5, shape_id=N + K)
    Wd = to_dev(W)
    for M in range(1, 9):
        x = synth.activations(M, K, seed=5, shape_id=N + K, tensor_id=M)
        ws = skg.split_k_workspace(M, N, K)
        y = skg.gemm_split_k(to_dev(x), Wd, ws)
        check(y, x, W, f"({N},{K}) M={M}")


# ---------------------------------------------------------------------------
# counters return to zero: repeated calls, shape changes, graph replays
# ---------------------------------------------------------------------------

def test_workspace_reused_across_calls_and_shapes(skg):
    """One workspace sized for the largest call serves a run of calls with other
    N, M and S, each checked against the oracle, then the first call again."""
    K = 4096
    big = skg.split_k_workspace(8, 4096, K, split_plan(skg, 64, 1, 1, 8))
    cases = [(4096, 8, 8, 1), (1000, 3, 4, 2), (77, 1, 2, 4), (4096, 2, 8, 1), (2049, 8, 4, 2),
             (4096, 8, 8, 1)]
    first = None
    for i, (N, M, S, chunks) in enumerate(cases):
        plan = split_plan(skg, 64, chunks, 1, S)
        assert S * 64 * 8 * chunks == K
        assert skg.skinny_gemm_split_k_workspace_bytes(M, N, K, plan) <= big.numel()
        W = synth.weights(N, K, seed=6, shape_id=N, tensor_id=1)
        x = synth.activations(M, K, seed=6, shape_id=N, tensor_id=M)
        y = skg.gemm_split_k(to_dev(x), to_dev(W), big, plan=plan)
        check(y, x, W, f"call {i}: N={N} M={M} S={S}")
        if i == 0:
            first = to_host(y)
        if i == len(cases) - 1:
            assert np.array_equal(to_host(y), first)
    torch.cuda.synchronize()


def test_repeated_calls_are_deterministic(skg):
    N, K, M = 2048, 4096, 4
    W = to_dev(synth.weights(N, K, seed=7))
    x = to_dev(synth.activations(M, K, seed=7))
    ws = skg.split_k_workspace(M, N, K)
    ys = [to_host(skg.gemm_split_k(x, W, ws)) for _ in range(5)]
    for y in ys[1:]:
        assert np.array_equal(y, ys[0])


def test_graph_replay(skg):
    """Captured once, replayed three times with the output poisoned before each
    replay and eager work between replays: every replay gives the eager bits."""
    N, K, M = 4096, 8192, 4
    W = synth.weights(N, K, seed=8)
    x = synth.activations(M, K, seed=8)
    Wd, xd = to_dev(W), to_dev(x)
    ws = skg.split_k_workspace(M, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    skg.gemm_split_k(xd, Wd, ws, out=y)
    torch.cuda.synchronize()
    eager = to_host(y)
    check(y, x, W, "eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            skg.gemm_split_k(xd, Wd, ws, out=y)
    torch.cuda.current_stream().wait_stream(s)
    other = skg.split_k_workspace(2, 1000, K)
    for rep in range(3):
        nan_fill(y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), eager), f"replay {rep}"
        # eager split-K work on another workspace between replays
        skg.gemm_split_k(xd[:2], Wd[:1000], other)
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# refusals that need a device pointer to be meaningful
# ---------------------------------------------------------------------------

def test_refusals(skg):
    L = skg.lib()
    N, K, M = 1024, 4096, 2
    W = to_dev(synth.weights(N, K, seed=9))
    x = to_dev(synth.activations(M, K, seed=9))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    plan = skg.skinny_gemm_split_k_default_plan(M, N, K)
    need = skg.skinny_gemm_split_k_workspace_bytes(M, N, K, plan)
    ws = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    import ctypes

    p = ctypes.byref(plan)
    call = L.skinny_gemm_bf16_split_k
    E = skg.SKINNY_ERR_INVALID_ARG
    assert call(x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K, p, ws.data_ptr(), need, s) == 0
    assert call(x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K, p, ws.data_ptr(), need - 4, s) == E
    assert call(x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K, p, None, need, s) == E
    assert call(x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K, p, ws.data_ptr() + 16, need, s) == E
    # workspace over y, over W
    assert call(x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K, p, y.data_ptr(), need, s) == E
    assert call(x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K, p, W.data_ptr(), need, s) == E
    # K not S * slice, misaligned x, M out of range
    assert call(x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, 2048, p, ws.data_ptr(), need, s) == E
    assert call(x.data_ptr() + 2, W.data_ptr(), y.data_ptr(), M, N, K - 8, None, ws.data_ptr(), need, s) == E
    assert call(x.data_ptr(), W.data_ptr(), y.data_ptr(), 9, N, K, None, ws.data_ptr(), need, s) == E
    torch.cuda.synchronize()
    check(y, to_host(x), to_host(W), "the accepted call")


def test_many_back_to_back_calls_match_in_block(skg):
    """300 split-K calls queued back to back on one workspace, S = 2..16 with many
    tiles (every block of a tile on a different XCD), each compared bit for bit with
    the in-block plan of the same slices: a partial read before it is visible, or a
    counter left behind, would show as a mismatch."""
    K = 4096
    cases = []
    for chunks, S in ((4, 2), (2, 4)):
        for N in (4096, 1000):
            W = to_dev(synth.weights(N, K, seed=10, shape_id=N, tensor_id=S))
            x = to_dev(synth.activations(4, K, seed=10, shape_id=N, tensor_id=S))
            ref = skg.gemm(x, W, plan=fixed_plan(skg, 64, chunks, 1, S, tpb=64 * S))
            cases.append((x, W, split_plan(skg, 64, chunks, 1, S, tpb=64), to_host(ref)))
    # S = 8 and 16 have no in-block twin at K = 4096: the reference is the oracle-checked
    # first call
    ws = skg.split_k_workspace(4, 4096, K, split_plan(skg, 32, 1, 1, 16))
    for lanes, S, N in ((64, 8, 4096), (32, 16, 2048)):
        W = synth.weights(N, K, seed=11, shape_id=S)
        x = synth.activations(3, K, seed=11, shape_id=S)
        p = split_plan(skg, lanes, 1, 1, S)
        y = skg.gemm_split_k(to_dev(x), to_dev(W), ws, plan=p)
        check(y, x, W, f"S={S}")
        cases.append((to_dev(x), to_dev(W), p, to_host(y)))
    outs = []
    for rep in range(300):
        x, W, plan, ref = cases[rep % len(cases)]
        outs.append((skg.gemm_split_k(x, W, ws, plan=plan), ref))
    torch.cuda.synchronize()
    for i, (y, ref) in enumerate(outs):
        assert np.array_equal(to_host(y), ref), f"call {i}"


def test_concurrent_streams_with_own_workspaces(skg):
    """Four host threads, each on its own stream with its own workspace, run split-K
    calls at the same time (the use the contract allows): every output matches the
    oracle-checked reference bit for bit."""
    import threading

    K = 4096
    refs, jobs = [], []
    for t in range(4):
        N, M = 2048 + 512 * t, 1 + t
        W = synth.weights(N, K, seed=12, shape_id=t)
        x = synth.activations(M, K, seed=12, shape_id=t)
        Wd, xd = to_dev(W), to_dev(x)
        y = skg.gemm_split_k(xd, Wd, skg.split_k_workspace(M, N, K))
        check(y, x, W, f"thread {t} reference")
        refs.append(to_host(y))
        jobs.append((xd, Wd, skg.split_k_workspace(M, N, K), torch.cuda.Stream()))
    torch.cuda.synchronize()
    outs = [[] for _ in jobs]
    errors = []

    def work(i):
        try:
            xd, Wd, ws, stream = jobs[i]
            with torch.cuda.stream(stream):
                for _ in range(50):
                    outs[i].append(skg.gemm_split_k(xd, Wd, ws))
            stream.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, ys in enumerate(outs):
        assert len(ys) == 50
        for y in ys:
            assert np.array_equal(to_host(y), refs[i]), f"thread {i}"
