"""Parity of the HIP path with the CPU oracle on an MI355X (gfx950).

Every call goes through the C ABI (the ctypes binding passes raw device
pointers and torch's current stream). The acceptance bar: per element
|y - y_ref| <= 1e-2 * sum_k |x_k W_nk| + 1e-6, per output row cosine >= 0.99999,
and additionally the float64 rule of vLLM PR #65306 (SM90 skinny GEMM plans),
section Validation: |y - ref64| <= 7.5e-5 + 2^-8 |ref64|
(oracle/accept.py). Exact cases (zero, identity, one-hot, small integers,
rounding ties) must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

CONFIG_SHAPES = [(4096, 1024), (12576, 4096), (4096, 4096), (2048, 4096), (8192, 1536),
                 (4096, 8192)]
LM_HEAD = (77440, 4096)


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


def check(y_dev, x, W, rows=None, label=""):
    yb = to_host(y_dev)
    if rows is None:
        yr, ref, mag = oracle.gemm(x, W)
        res = oracle.acceptance(yb, yr, ref, mag)
    else:
        yr, ref, mag = oracle.gemm_rows(x, W, rows)
        res = oracle.acceptance(yb[:, rows], yr, ref, mag, check_cosine=False)
    assert res["pass"], f"{label}: {res}"
    return res


def fixed_k(p):
    return p.k_split * p.lanes_per_row * 8 * p.chunks


def variant_K(p):
    if p.kind == 1:
        return [fixed_k(p)]
    if p.kind == 2:
        return [8, 1000, 4096 + 8]
    if p.kind == 4:
        unit = 128 * p.k_split * p.chunks
        return [unit, 3 * unit]
    return [1, 13, 1001]


def plan_runs_k(p, K):
    if p.kind == 1:
        return fixed_k(p) == K
    if p.kind == 4:
        return K % (128 * p.k_split) == 0 and (K // (128 * p.k_split)) % p.chunks == 0
    return True


def rows_per_tile(p, tpb=None):
    tpb = tpb or p.threads_per_block
    return (tpb // 64 // p.k_split) * p.rows_per_wave * (64 // p.lanes_per_row)


# ---------------------------------------------------------------------------
# every compiled variant, every M, several tiles plus a ragged tail
# ---------------------------------------------------------------------------

def _variant_cases():
    import bf16_skinny_gemm_amd as m

    try:
        vs = m.variants()
    except Exception:  # library missing: collected as one failing case
        return [pytest.param(None, id="no-library")]
    return [pytest.param(v, id=f"v{i}-k{v.kind}-l{v.lanes_per_row}-c{v.chunks}-r{v.rows_per_wave}"
                                f"-s{v.k_split}-nt{v.nontemporal}-x{v.x_in_lds}-p{v.prefetch}")
            for i, v in enumerate(vs)]


@pytest.mark.parametrize("plan", _variant_cases())
def test_every_variant(skg, plan):
    assert plan is not None, "library missing"
    ran = 0
    for K in variant_K(plan):
        for M in range(1, 9):
            tile = rows_per_tile(plan)
            N = 3 * tile + 5  # four tiles, the last one ragged
            x = synth.activations(M, K, seed=0, shape_id=K, tensor_id=M)
            W = synth.weights(N, K, seed=0, shape_id=K, tensor_id=1)
            xd, Wd = to_dev(x), to_dev(W)
            # the plan's own grid (one tile per block), then one block looping over all
            # four tiles and three blocks taking two, one and one: every prefetch mode
            # runs its multi-tile loop, odd and even trip counts
            for grid in (plan.grid_blocks, 1, 3):
                q = skg.Plan.from_dict({**plan.as_dict(), "grid_blocks": grid})
                try:
                    y = skg.gemm(xd, Wd, plan=q)
                except skg.SkinnyError as e:
                    # this M exceeds the variant's register budget (fixed-K) or the 4 rows
                    # of the MFMA A operand, or x of this K does not fit in a block's LDS
                    # (kinds that stage x there)
                    assert e.status == skg.SKINNY_ERR_UNSUPPORTED, str(e)
                    assert (plan.kind == 1 or (plan.kind == 4 and M > 4)
                            or M * K * 2 > 64 * 1024), str(e)
                    break
                torch.cuda.synchronize()
                check(y, x, W, label=f"{q} M={M} N={N} K={K}")
                ran += 1
    assert ran > 0, f"no M runs on {plan}"


@pytest.mark.parametrize("tpb", [64, 128, 512])
def test_block_sizes_and_persistent_grid(skg, tpb):
    """Launch-time knobs: block size, and persistent grids smaller than the tile
    count (6 tiles over 2 or 4 blocks: three, or two and one, tiles per block)."""
    for K in (1024, 4096):
        for p in skg.variants():
            if p.kind != 1 or fixed_k(p) != K or (tpb // 64) % p.k_split:
                continue
            for grid in (0, 2, 4):
                q = skg.Plan.from_dict({**p.as_dict(), "threads_per_block": tpb, "grid_blocks": grid})
                M = 2
                N = 5 * rows_per_tile(q) + 3
                x = synth.activations(M, K, seed=1, shape_id=tpb)
                W = synth.weights(N, K, seed=1, shape_id=tpb)
                y = skg.gemm(to_dev(x), to_dev(W), plan=q)
                torch.cuda.synchronize()
                check(y, x, W, label=f"{q}")


# ---------------------------------------------------------------------------
# the decode shapes at full size through the default entry point
# ---------------------------------------------------------------------------

def table_shapes():
    """Every (N, K) of the generated plan table, with the token counts it tunes."""
    import os
    import re

    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "bf16_skinny_gemm_amd", "csrc", "plans_gfx950.inc")
    cells = {}
    for n, k, m in re.findall(r"^\{(\d+), (\d+), (\d+), \{", open(path).read(), re.M):
        cells.setdefault((int(n), int(k)), []).append(int(m))
    return sorted(cells.items())


@pytest.mark.parametrize("shape,ms", [pytest.param(s, m, id=f"{s[0]}x{s[1]}")
                                      for s, m in table_shapes() if s != LM_HEAD])
def test_table_shapes_full(skg, shape, ms):
    """Every (N, K, M) the plan table tunes, at its full size through the default
    entry point (the table's plan, its grid), the whole output against the oracle:
    G1 per element, G2 per row, S1. The K = 128 shapes are the paired projections'
    and also run as pairs."""
    N, K = shape
    assert sorted(ms) == list(range(1, 9)), f"table rows of {shape}: {ms}"
    W = synth.weights(N, K, seed=0, shape_id=N * 7 + K, tensor_id=1)
    Wd = to_dev(W)
    W1 = W1d = None
    if K == 128:
        W1 = synth.weights(N, K, seed=0, shape_id=N * 7 + K, tensor_id=2)
        W1d = to_dev(W1)
    for M in ms:
        x = synth.activations(M, K, seed=0, shape_id=N * 7 + K, tensor_id=0)
        xd = to_dev(x)
        plan, tuned = skg.skinny_gemm_get_plan(N, K, M)
        assert tuned, f"({N},{K}) M={M} has no table row"
        y = skg.gemm(xd, Wd)
        torch.cuda.synchronize()
        check(y, x, W, label=f"N={N} K={K} M={M} {plan}")
        if W1 is not None:
            y0, y1 = skg.gemm_pair(xd, Wd, W1d)
            torch.cuda.synchronize()
            check(y0, x, W, label=f"pair y0 N={N} K={K} M={M}")
            check(y1, x, W1, label=f"pair y1 N={N} K={K} M={M}")


@pytest.mark.parametrize("M", range(1, 9))
def test_lm_head_full(skg, M):
    """(77440, 4096), 634 MB: the whole output of every row against the oracle,
    G1 per element, G2 (cosine >= 0.99999) per output row, S1."""
    N, K = LM_HEAD
    W = _lm_head_weight()
    x = synth.activations(M, K, seed=0, shape_id=5, tensor_id=0)
    y = skg.gemm(to_dev(x), _lm_head_weight_dev())
    torch.cuda.synchronize()
    res = check(y, x, W, label=f"lm_head M={M}")
    assert res["min_cos"] >= 0.99999 and res["n"] == M * N


_LM = {}


def _lm_head_weight():
    if "host" not in _LM:
        _LM["host"] = synth.weights(*LM_HEAD, seed=0, shape_id=5, tensor_id=1)
    return _LM["host"]


def _lm_head_weight_dev():
    if "dev" not in _LM:
        _LM["dev"] = to_dev(_lm_head_weight())
    return _LM["dev"]


def test_pair_shape(skg):
    """Paired (4096, 128) weights on one x: both outputs match the oracle, and each
    equals a single call with the same plan bit for bit."""
    N, K = 4096, 128
    W0 = synth.weights(N, K, seed=0, shape_id=6, tensor_id=1)
    W1 = synth.weights(N, K, seed=0, shape_id=6, tensor_id=2)
    W0d, W1d = to_dev(W0), to_dev(W1)
    for M in range(1, 9):
        x = synth.activations(M, K, seed=0, shape_id=6, tensor_id=0)
        xd = to_dev(x)
        y0, y1 = skg.gemm_pair(xd, W0d, W1d)
        torch.cuda.synchronize()
        check(y0, x, W0, label=f"pair y0 M={M}")
        check(y1, x, W1, label=f"pair y1 M={M}")
        plan, _ = skg.skinny_gemm_get_plan(N, K, M)
        s0 = skg.gemm(xd, W0d, plan=plan)
        s1 = skg.gemm(xd, W1d, plan=plan)
        assert torch.equal(y0.view(torch.int16), s0.view(torch.int16))
        assert torch.equal(y1.view(torch.int16), s1.view(torch.int16))


def test_pair_all_variants_match_singles(skg):
    M, K = 3, 128
    x = synth.activations(M, K, seed=2)
    for p in skg.variants():
        if not plan_runs_k(p, K):
            continue
        N = 2 * rows_per_tile(p) + 9
        W0 = synth.weights(N, K, seed=2, tensor_id=1)
        W1 = synth.weights(N, K, seed=2, tensor_id=2)
        xd, W0d, W1d = to_dev(x), to_dev(W0), to_dev(W1)
        y0, y1 = skg.gemm_pair(xd, W0d, W1d, plan=p)
        s0 = skg.gemm(xd, W0d, plan=p)
        s1 = skg.gemm(xd, W1d, plan=p)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), s0.view(torch.int16)), p
        assert torch.equal(y1.view(torch.int16), s1.view(torch.int16)), p
        check(y1, x, W1, label=f"pair {p}")


# ---------------------------------------------------------------------------
# exact cases: bit for bit
# ---------------------------------------------------------------------------

def _exact(skg, x, W, label):
    y = skg.gemm(to_dev(x), to_dev(W))
    torch.cuda.synchronize()
    yr, _, _ = oracle.gemm(x, W)
    np.testing.assert_array_equal(to_host(y), yr, err_msg=label)


@pytest.mark.parametrize("K", [128, 1024, 1536, 4096, 8192, 1000, 37])
def test_exact_special_cases(skg, K):
    g = np.random.default_rng(K)
    for M in (1, 4, 8):
        x = synth.activations(M, K, seed=20, shape_id=K)
        # zero weight
        _exact(skg, x, np.zeros((70, K), np.uint16), f"zero K={K}")
        # one-hot rows
        N = 300
        perm = g.integers(0, K, size=N)
        W = np.zeros((N, K), np.uint16)
        W[np.arange(N), perm] = synth.BF16_ONE
        _exact(skg, x, W, f"one-hot K={K} M={M}")
        # small integers, |sum| <= 256 so every partial sum is exact in float32
        xi = synth.small_int_bf16((M, K), -1, 1, g)
        Wi = synth.small_int_bf16((N, K), -1, 1, g)
        if K > 256:
            Wi[:, 256:] = 0
        _exact(skg, xi, Wi, f"small-int K={K} M={M}")
    # identity (square)
    if K <= 4096:
        x = synth.activations(2, K, seed=21, shape_id=K)
        W = np.zeros((K, K), np.uint16)
        W[np.arange(K), np.arange(K)] = synth.BF16_ONE
        _exact(skg, x, W, f"identity K={K}")


@pytest.mark.parametrize("K", [2, 1024, 4096])
def test_rounding_mode_ties(skg, K):
    """x.W = 1 + 2^-8 and 1 + 3*2^-8 are exact float32 sums halfway between bfloat16
    neighbours: round-to-nearest-even gives 1.0 and 1 + 2^-6; truncation or
    round-half-up gives a different answer on one of the two."""
    def bits(v):
        return synth.f32_to_bf16_bits(np.array(v, np.float32))

    x = np.zeros((2, K), np.uint16)
    x[0, :2] = bits([1.0, 2.0 ** -8])
    x[1, :2] = bits([1.0, 3 * 2.0 ** -8])
    W = np.zeros((4, K), np.uint16)
    W[:, :2] = synth.BF16_ONE
    y = to_host(skg.gemm(to_dev(x), to_dev(W)))
    assert np.all(y[0] == 0x3F80) and np.all(y[1] == 0x3F82), [hex(v) for v in y.ravel()]
    # negative side
    W[:, :2] = bits([-1.0, -1.0])
    y = to_host(skg.gemm(to_dev(x), to_dev(W)))
    assert np.all(y[0] == 0xBF80) and np.all(y[1] == 0xBF82)
    # M = 8: the two ties alternate over all eight rows of the output
    x8 = np.zeros((8, K), np.uint16)
    x8[0::2] = x[0]
    x8[1::2] = x[1]
    W[:, :2] = synth.BF16_ONE
    y = to_host(skg.gemm(to_dev(x8), to_dev(W)))
    assert np.all(y[0::2] == 0x3F80) and np.all(y[1::2] == 0x3F82), [hex(v) for v in y.ravel()]


# ---------------------------------------------------------------------------
# invariants: graph replay, determinism, no stray writes
# ---------------------------------------------------------------------------

def test_graph_replay_bitwise(skg):
    """Every entry point captured in one graph (single, pair, strided pair over a
    merged activation, float32 output) replays bit for bit like the eager calls, with
    eager work between replays."""
    cases = [(4096, 1024, 1), (12576, 4096, 4), (4096, 128, 2), (4096, 4096, 8)]
    for (N, K, M) in cases:
        xm = to_dev(synth.activations(M, 2 * K, seed=30))   # merged [M, 2K]
        x = xm[:, :K].contiguous()
        W = to_dev(synth.weights(N, K, seed=30))
        W1 = to_dev(synth.weights(N, K, seed=31))
        eager = skg.gemm(x, W)
        e0, e1 = skg.gemm_pair(x, W, W1)
        es0, es1 = skg.gemm_pair_strided(xm[:, :K], xm[:, K:], W, W1)
        e32 = skg.gemm(x, W, out_dtype=torch.float32)
        out = torch.empty_like(eager)
        o0, o1 = torch.empty_like(e0), torch.empty_like(e1)
        merged = torch.empty((M, 2 * N), dtype=torch.bfloat16, device="cuda")
        s0, s1 = merged[:, :N], merged[:, N:]
        o32 = torch.empty_like(e32)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            skg.gemm(x, W, out=out)  # warm the stream before capture
            with torch.cuda.graph(g, stream=s):
                skg.gemm(x, W, out=out)
                skg.gemm_pair(x, W, W1, out0=o0, out1=o1)
                skg.gemm_pair_strided(xm[:, :K], xm[:, K:], W, W1, out0=s0, out1=s1)
                skg.gemm(x, W, out=o32, out_dtype=torch.float32)
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(4):
            for t in (out, o0, o1, merged, o32):
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), (N, K, M, rep)
            assert torch.equal(o0.view(torch.int16), e0.view(torch.int16))
            assert torch.equal(o1.view(torch.int16), e1.view(torch.int16))
            assert torch.equal(s0.contiguous().view(torch.int16), es0.contiguous().view(torch.int16))
            assert torch.equal(s1.contiguous().view(torch.int16), es1.contiguous().view(torch.int16))
            assert torch.equal(o32.view(torch.int32), e32.view(torch.int32))
            _ = skg.gemm(x, W)  # eager work between replays
        del g


def test_graph_dependent_chain_runs_in_order(skg):
    """Calls captured into one graph on one stream run in stream order: a chain whose
    call i+1 reads the first M*K outputs of call i (every output set to NaN before
    each replay, so a call that ran early would read NaN) replays bit for bit like the
    same calls run one at a time with the device synchronised after each. The decode
    benchmark times its calls on this ordering."""
    N, K = 4096, 1024
    for M in (1, 4):
        Ws = [to_dev(synth.weights(N, K, seed=40, tensor_id=i)) for i in range(6)]
        x0 = to_dev(synth.activations(M, K, seed=41))
        outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in Ws]
        xs = [x0] + [o.view(-1)[:M * K].view(M, K) for o in outs[:-1]]

        def chain():
            for x, W, y in zip(xs, Ws, outs):
                skg.gemm(x, W, out=y)

        ref = []
        for x, W in zip(xs, Ws):
            y = skg.gemm(x, W)
            torch.cuda.synchronize()
            ref.append(y)
            if len(ref) < len(Ws):
                # the next eager call reads this output through xs
                outs[len(ref) - 1].copy_(y)
                torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            chain()
            with torch.cuda.graph(g, stream=s):
                chain()
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(3):
            for o in outs:
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for i, (o, r) in enumerate(zip(outs, ref)):
                assert torch.equal(o.view(torch.int16), r.view(torch.int16)), (M, rep, i)
        del g


def test_concurrent_host_threads(skg):
    """Entry points called from several host threads at once, each on its own stream,
    through plans and M values whose lazily filled host caches (occupancy, static LDS,
    raised LDS limits) are first touched concurrently: every result meets the bar."""
    import threading

    cases = []
    for i, (N, K, M) in enumerate([(1000, 4096, 1), (777, 4096, 8), (513, 1024, 3),
                                   (2048, 8192, 6), (300, 1536, 2), (129, 128, 7),
                                   (4096, 4096, 5), (96, 1000, 4)]):
        x = synth.activations(M, K, seed=140, shape_id=i)
        W = synth.weights(N, K, seed=140, shape_id=i)
        cases.append((x, W, to_dev(x), to_dev(W)))
    plans = [p for p in skg.variants() if p.kind in (1, 2)]
    results, errors = {}, []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for r in range(6):
                    x, W, xd, Wd = cases[(t + r) % len(cases)]
                    K = x.shape[1]
                    # alternate the table plan with explicit grids of compiled variants
                    cand = [p for p in plans if plan_runs_k(p, K)]
                    plan = None
                    if r % 2 and cand:
                        plan = skg.Plan.from_dict({**cand[(7 * t + r) % len(cand)].as_dict(),
                                                   "grid_blocks": 1 + (t + r) % 5})
                    try:
                        y = skg.gemm(xd, Wd, plan=plan)
                    except skg.SkinnyError as e:  # this M beyond the variant's budget
                        assert e.status == skg.SKINNY_ERR_UNSUPPORTED, str(e)
                        y = skg.gemm(xd, Wd)
                    s.synchronize()
                    results[(t, r)] = (to_host(y), (t + r) % len(cases))
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    assert len(results) == 48
    for (t, r), (yb, ci) in results.items():
        x, W, _, _ = cases[ci]
        yr, ref, mag = oracle.gemm(x, W)
        res = oracle.acceptance(yb, yr, ref, mag)
        assert res["pass"], f"thread {t} call {r}: {res}"


def test_deterministic(skg):
    N, K, M = 8192, 1536, 4
    x = to_dev(synth.activations(M, K, seed=40))
    W = to_dev(synth.weights(N, K, seed=40))
    ref = skg.gemm(x, W)
    for p in skg.variants():
        if not plan_runs_k(p, K):
            continue
        if p.kind == 1:
            try:
                a = skg.gemm(x, W, plan=p)
            except skg.SkinnyError:
                continue
        else:
            a = skg.gemm(x, W, plan=p)
        b = skg.gemm(x, W, plan=p)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), p
    again = skg.gemm(x, W)
    assert torch.equal(ref.view(torch.int16), again.view(torch.int16))


def test_same_reduction_order_same_bits(skg):
    """Plans that differ only in rows per wave, block size, grid or the cache hint
    sum in the same order, so they give the same bits."""
    N, K, M = 4096, 4096, 2
    x = to_dev(synth.activations(M, K, seed=41))
    W = to_dev(synth.weights(N, K, seed=41))
    groups = {}
    for p in skg.variants():
        if p.kind != 1 or fixed_k(p) != K:
            continue
        key = (p.lanes_per_row, p.chunks, p.k_split)
        for tpb in (256, 512):
            q = skg.Plan.from_dict({**p.as_dict(), "threads_per_block": tpb, "grid_blocks": 0})
            try:
                y = skg.gemm(x, W, plan=q)
            except skg.SkinnyError:
                continue
            groups.setdefault(key, []).append((q, y))
    assert groups
    for key, ys in groups.items():
        for q, y in ys[1:]:
            assert torch.equal(y.view(torch.int16), ys[0][1].view(torch.int16)), (key, q)


def test_guard_band(skg):
    """Outputs are written only inside y: sentinels around it stay untouched, for the
    table's plans, one explicit plan of each vector family at a ragged N, and the
    float32 output."""
    fams = {}
    for p in skg.variants():
        if p.kind in (1, 2, 4) and p.kind not in fams and plan_runs_k(p, 4096):
            fams[p.kind] = p
    cases = [(4096 + 3, 1024, 3, None), (300, 128, 4, None), (77, 1000, 2, None),
             (65, 13, 1, None), (129, 4096, 8, None)]
    cases += [(4 * rows_per_tile(p) + 5, 4096, 3, p) for p in fams.values()]
    for (N, K, M, plan) in cases:
        for dt in (torch.bfloat16, torch.float32):
            pad = 4096
            buf = torch.full((M * N + 2 * pad,), -7.0, dtype=dt, device="cuda")
            y = buf[pad:pad + M * N].view(M, N)
            x = synth.activations(M, K, seed=50, shape_id=N)
            W = synth.weights(N, K, seed=50, shape_id=N)
            skg.gemm(to_dev(x), to_dev(W), out=y, plan=plan, out_dtype=dt)
            torch.cuda.synchronize()
            assert torch.all(buf[:pad] == -7.0) and torch.all(buf[pad + M * N:] == -7.0), \
                (N, K, M, plan, dt)
            if dt == torch.bfloat16:
                check(y, x, W, label=f"guard N={N} K={K} M={M} {plan}")
            else:
                check_f32(y, x, W, label=f"guard f32 N={N} K={K} M={M} {plan}")


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 8), (1, 1), (2, 4096), (63, 128), (64, 128), (65, 128),
                                 (5, 8200), (3, 520), (129, 1536), (1000, 24), (7, 16384)])
def test_edges(skg, N, K):
    for M in range(1, 9):
        x = synth.activations(M, K, seed=60, shape_id=N)
        W = synth.weights(N, K, seed=60, shape_id=N)
        y = skg.gemm(to_dev(x), to_dev(W))
        torch.cuda.synchronize()
        check(y, x, W, label=f"edge N={N} K={K} M={M}")


def test_misaligned_pointers(skg):
    """Views that start one element in: x and W lose 16-byte alignment, the library
    takes its element-wise path and is still correct."""
    M, N, K = 2, 333, 1024
    x = synth.activations(M, K + 1, seed=61)[:, 1:].copy()
    W = synth.weights(N, K + 1, seed=61)[:, 1:].copy()
    xb = torch.empty(M * K + 1, dtype=torch.bfloat16, device="cuda")
    Wb = torch.empty(N * K + 1, dtype=torch.bfloat16, device="cuda")
    xb[1:] = to_dev(x).view(-1)
    Wb[1:] = to_dev(W).view(-1)
    xv = xb[1:].view(M, K)
    Wv = Wb[1:].view(N, K)
    assert xv.data_ptr() % 16 != 0
    y = skg.gemm(xv, Wv)
    torch.cuda.synchronize()
    check(y, x, W, label="misaligned")
    y0, y1 = skg.gemm_pair(xv, Wv, Wv)
    torch.cuda.synchronize()
    check(y0, x, W, label="misaligned pair")
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def test_k_zero_and_empty(skg):
    x = torch.empty((3, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((50, 0), dtype=torch.bfloat16, device="cuda")
    y = torch.full((3, 50), 5.0, dtype=torch.bfloat16, device="cuda")
    skg.gemm(x, W, out=y)
    torch.cuda.synchronize()
    assert torch.all(y.view(torch.int16) == 0)  # +0, the empty sum
    y0 = torch.full((3, 50), 5.0, dtype=torch.bfloat16, device="cuda")
    y1 = torch.full((3, 50), 5.0, dtype=torch.bfloat16, device="cuda")
    skg.gemm_pair(x, W, W, out0=y0, out1=y1)
    torch.cuda.synchronize()
    assert torch.all(y0.view(torch.int16) == 0) and torch.all(y1.view(torch.int16) == 0)
    # N == 0 and M == 0: nothing to do
    e = skg.gemm(torch.empty((2, 64), dtype=torch.bfloat16, device="cuda"),
                 torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert e.shape == (2, 0)
    e = skg.gemm(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                 torch.empty((10, 64), dtype=torch.bfloat16, device="cuda"))
    assert e.shape == (0, 10)


def test_rejects_m9(skg):
    with pytest.raises(skg.SkinnyError):
        skg.gemm(torch.zeros((9, 64), dtype=torch.bfloat16, device="cuda"),
                 torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda"))


def _robust_x(kind, M, K, shape_id, tensor_id=0):
    if kind == "outlier":
        return synth.outlier_activations(M, K, seed=70, shape_id=shape_id, tensor_id=tensor_id)
    if kind == "scaled_up":
        return synth.scaled_activations(M, K, 8, seed=70, shape_id=shape_id, tensor_id=tensor_id)
    if kind == "scaled_down":
        return synth.scaled_activations(M, K, -8, seed=70, shape_id=shape_id, tensor_id=tensor_id)
    return synth.sparse_activations(M, K, seed=70, shape_id=shape_id, tensor_id=tensor_id)


ROBUST_KINDS = ["outlier", "scaled_up", "scaled_down", "sparse"]


@pytest.mark.parametrize("kind", ROBUST_KINDS)
def test_robustness_inputs(skg, kind):
    """Input classes beyond normal (vLLM PR #65306, section Validation): outlier,
    scaled and sparse, on every single-GEMM shape of the decode projections
    (whole outputs; the LM head at M = 1 and 4), through the table's plans."""
    for (N, K) in CONFIG_SHAPES + [LM_HEAD]:
        W = synth.weights(N, K, seed=70, shape_id=N)
        Wd = to_dev(W)
        for M in ((1, 4) if (N, K) == LM_HEAD else (1, 2, 4, 8)):
            x = _robust_x(kind, M, K, N)
            y = skg.gemm(to_dev(x), Wd)
            torch.cuda.synchronize()
            check(y, x, W, label=f"{kind} N={N} K={K} M={M}")


@pytest.mark.parametrize("kind", ROBUST_KINDS)
def test_robustness_inputs_other_entry_points(skg, kind):
    """The same input classes through the paired, strided-pair, float32-output and
    split-K entry points."""
    N, K = 4096, 128
    W0, W1 = synth.weights(N, K, seed=71, tensor_id=1), synth.weights(N, K, seed=71, tensor_id=2)
    W0d, W1d = to_dev(W0), to_dev(W1)
    for M in (1, 4, 8):
        x = _robust_x(kind, M, K, 1, M)
        y0, y1 = skg.gemm_pair(to_dev(x), W0d, W1d)
        check(y0, x, W0, label=f"{kind} pair y0 M={M}")
        check(y1, x, W1, label=f"{kind} pair y1 M={M}")
        xm = _robust_x(kind, M, 2 * K, 2, M)
        xmd = to_dev(xm)
        z0, z1 = skg.gemm_pair_strided(xmd[:, :K], xmd[:, K:], W0d, W1d)
        check(z0, np.ascontiguousarray(xm[:, :K]), W0, label=f"{kind} strided y0 M={M}")
        check(z1, np.ascontiguousarray(xm[:, K:]), W1, label=f"{kind} strided y1 M={M}")
    N, K = 288, 4096  # the router gate, float32 outputs
    W = synth.weights(N, K, seed=72)
    for M in (1, 4, 8):
        x = _robust_x(kind, M, K, 3, M)
        y = skg.gemm(to_dev(x), to_dev(W), out_dtype=torch.float32)
        check_f32(y, x, W, label=f"{kind} f32out M={M}")
    N, K = 2048, 4096  # split-K, default plan
    W = synth.weights(N, K, seed=73)
    Wd = to_dev(W)
    for M in (1, 4, 8):
        x = _robust_x(kind, M, K, 4, M)
        y = skg.gemm_split_k(to_dev(x), Wd, skg.split_k_workspace(M, N, K))
        check(y, x, W, label=f"{kind} split-K M={M}")


def test_weight_beyond_4gib(skg):
    """A weight larger than 4 GiB (N = 270000, K = 8192): 64-bit row addressing.
    W is drawn on the GPU; the rows the oracle checks are copied back."""
    N, K, M = 270000, 8192, 2
    free, _ = torch.cuda.mem_get_info()
    if free < 12 * 2 ** 30:
        pytest.skip("not enough device memory")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(80)
    Wd = (torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32)
          * (1.0 / K ** 0.5)).to(torch.bfloat16)
    x = synth.activations(M, K, seed=80)
    y = skg.gemm(to_dev(x), Wd)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 64), np.arange(N - 512, N),
                           np.array([N // 2, 262144, 262145])]).astype(np.int64)
    W_rows = to_host(Wd[torch.from_numpy(rows).cuda()])
    yr, ref, mag = oracle.gemm(x, W_rows)
    res = oracle.acceptance(to_host(y)[:, rows], yr, ref, mag, check_cosine=False)
    assert res["pass"], res
    del Wd
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# float32-output form (router gate epilogue)
# ---------------------------------------------------------------------------

def check_f32(y_dev, x, W, rows=None, label=""):
    y = y_dev.cpu().numpy()
    assert y.dtype == np.float32
    yr, ref, mag = oracle.gemm_f32out(x, W, rows)
    yy = y if rows is None else y[:, rows]
    res = oracle.acceptance(yy, yr, ref, mag, check_cosine=rows is None)
    assert res["pass"], f"{label}: {res}"
    return res


@pytest.mark.parametrize("shape", [(288, 4096), (4096, 1024), (1000, 1536), (77, 1000), (33, 13),
                                   (4096, 128)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_f32_output(skg, shape):
    N, K = shape
    W = synth.weights(N, K, seed=90, shape_id=N)
    Wd = to_dev(W)
    for M in range(1, 9):
        x = synth.activations(M, K, seed=90, shape_id=N, tensor_id=M)
        xd = to_dev(x)
        y = skg.gemm(xd, Wd, out_dtype=torch.float32)
        torch.cuda.synchronize()
        check_f32(y, x, W, label=f"f32 N={N} K={K} M={M}")
        # the bf16 output is the same float32 sum rounded to nearest-even
        p, _ = skg.skinny_gemm_get_plan(N, K, M)
        if K % 8 == 0:
            yb = skg.gemm(xd, Wd, plan=p)
            y32 = skg.gemm(xd, Wd, plan=p, out_dtype=torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(yb.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


def test_f32_output_every_variant(skg):
    M = 2
    for p in skg.variants():
        K = variant_K(p)[0]
        N = 2 * rows_per_tile(p) + 3
        x = synth.activations(M, K, seed=91, shape_id=K)
        W = synth.weights(N, K, seed=91, shape_id=K)
        try:
            y = skg.gemm(to_dev(x), to_dev(W), plan=p, out_dtype=torch.float32)
        except skg.SkinnyError as e:
            assert e.status == skg.SKINNY_ERR_UNSUPPORTED and p.kind == 1, str(e)
            continue
        torch.cuda.synchronize()
        check_f32(y, x, W, label=f"f32 {p}")


def test_f32_output_exact_and_empty(skg):
    g = np.random.default_rng(92)
    K, N = 4096, 300
    xi = synth.small_int_bf16((4, K), -1, 1, g)
    Wi = synth.small_int_bf16((N, K), -1, 1, g)
    Wi[:, 256:] = 0  # |sum| <= 256: every partial sum exact in float32
    y = skg.gemm(to_dev(xi), to_dev(Wi), out_dtype=torch.float32).cpu().numpy()
    yr, _, _ = oracle.gemm_f32out(xi, Wi)
    np.testing.assert_array_equal(y, yr)
    # K == 0 writes +0.0f
    y = torch.full((3, 50), 5.0, dtype=torch.float32, device="cuda")
    skg.gemm(torch.empty((3, 0), dtype=torch.bfloat16, device="cuda"),
             torch.empty((50, 0), dtype=torch.bfloat16, device="cuda"), out=y,
             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(y.view(torch.int32) == 0)


def test_f32_output_rejects_misaligned(skg):
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    st = skg.lib().skinny_gemm_bf16_f32out(x.data_ptr(), W.data_ptr(), buf.data_ptr() + 2,
                                           1, 8, 64, None)
    assert st == skg.SKINNY_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(buf == 0)


# ---------------------------------------------------------------------------
# strided paired form: two halves of a merged activation, merged output
# ---------------------------------------------------------------------------

def _merged_case(M, N, K, seed, extra_cols=0):
    xm = synth.activations(M, 2 * K + extra_cols, seed=seed, shape_id=K, tensor_id=0)
    W0 = synth.weights(N, K, seed=seed, shape_id=K, tensor_id=1)
    W1 = synth.weights(N, K, seed=seed, shape_id=K, tensor_id=2)
    return xm, W0, W1


@pytest.mark.parametrize("N,K", [(4096, 128), (2048, 128), (300, 1024), (129, 1536)])
def test_pair_strided_merged(skg, N, K):
    for M in range(1, 9):
        xm, W0, W1 = _merged_case(M, N, K, seed=100 + M)
        xmd = to_dev(xm)
        W0d, W1d = to_dev(W0), to_dev(W1)
        y0, y1 = skg.gemm_pair_strided(xmd[:, :K], xmd[:, K:], W0d, W1d)
        torch.cuda.synchronize()
        x0 = np.ascontiguousarray(xm[:, :K])
        x1 = np.ascontiguousarray(xm[:, K:])
        check(y0.contiguous(), x0, W0, label=f"strided y0 M={M} N={N} K={K}")
        check(y1.contiguous(), x1, W1, label=f"strided y1 M={M} N={N} K={K}")
        # identical bits to two single calls with the same plan on contiguous inputs
        plan, _ = skg.skinny_gemm_get_plan(N, K, M)
        s0 = skg.gemm(to_dev(x0), W0d, plan=plan)
        s1 = skg.gemm(to_dev(x1), W1d, plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(y0.contiguous().view(torch.int16), s0.view(torch.int16))
        assert torch.equal(y1.contiguous().view(torch.int16), s1.view(torch.int16))


def test_pair_strided_every_variant(skg):
    M = 3
    for p in skg.variants():
        K = variant_K(p)[0]
        N = 2 * rows_per_tile(p) + 5
        xm, W0, W1 = _merged_case(M, N, K, seed=110)
        xmd = to_dev(xm)
        try:
            y0, y1 = skg.gemm_pair_strided(xmd[:, :K], xmd[:, K:], to_dev(W0), to_dev(W1), plan=p)
        except skg.SkinnyError as e:
            assert e.status == skg.SKINNY_ERR_UNSUPPORTED, str(e)
            continue
        torch.cuda.synchronize()
        check(y0.contiguous(), np.ascontiguousarray(xm[:, :K]), W0, label=f"strided y0 {p}")
        check(y1.contiguous(), np.ascontiguousarray(xm[:, K:]), W1, label=f"strided y1 {p}")


def test_kda_gate_chain_merged_fa_ga_then_strided_fb_gb(skg):
    """The KDA gate projections as two launches: one GEMV over the stacked f_a/g_a
    weight (2r rows) writes the merged [M, 2r] activation, whose two halves feed the
    strided f_b/g_b pair (ldx = 2r) (LMDeploy PR #4968, Optimizations: merge f_a/g_a,
    batch f_b/g_b; vLLM PR #57617, "Controlled follow-up": the strided view of the
    merged output). The r = 128 width is f_b/g_b's K; the hidden size 4096 is the
    KDA projections' K. Stage 1 is checked against the oracle; stage 2 against the
    oracle applied to stage 1's own bf16 output, so each launch meets the bar alone."""
    K, r, N = 4096, 128, 4096
    for M in (1, 2, 3, 4):
        x = synth.activations(M, K, seed=130, shape_id=K, tensor_id=M)
        Wa = synth.weights(2 * r, K, seed=130, shape_id=K, tensor_id=1)  # f_a rows, then g_a rows
        Wf = synth.weights(N, r, seed=130, shape_id=r, tensor_id=2)
        Wg = synth.weights(N, r, seed=130, shape_id=r, tensor_id=3)
        ya = skg.gemm(to_dev(x), to_dev(Wa))
        y0, y1 = skg.gemm_pair_strided(ya[:, :r], ya[:, r:], to_dev(Wf), to_dev(Wg))
        torch.cuda.synchronize()
        check(ya, x, Wa, label=f"merged f_a/g_a M={M}")
        ya_h = to_host(ya)
        check(y0.contiguous(), np.ascontiguousarray(ya_h[:, :r]), Wf, label=f"f_b M={M}")
        check(y1.contiguous(), np.ascontiguousarray(ya_h[:, r:]), Wg, label=f"g_b M={M}")


def test_pair_strided_odd_stride_and_guard(skg):
    """A row stride that breaks 16-byte alignment (element-wise path), separate
    outputs, and a merged output whose gap columns must stay untouched."""
    M, N, K = 4, 333, 128
    xm, W0, W1 = _merged_case(M, N, K, seed=120, extra_cols=1)  # ldx = 2K + 1
    xmd = to_dev(xm)
    y0, y1 = skg.gemm_pair_strided(xmd[:, :K], xmd[:, K:2 * K], to_dev(W0), to_dev(W1))
    torch.cuda.synchronize()
    check(y0.contiguous(), np.ascontiguousarray(xm[:, :K]), W0, label="odd stride y0")
    check(y1.contiguous(), np.ascontiguousarray(xm[:, K:2 * K]), W1, label="odd stride y1")
    # merged output with a guard column block between and after the halves
    xm, W0, W1 = _merged_case(M, N, K, seed=121)
    xmd = to_dev(xm)
    big = torch.full((M, 3 * N + 7), -3.0, dtype=torch.bfloat16, device="cuda")
    o0, o1 = big[:, :N], big[:, N + 7:2 * N + 7]
    skg.gemm_pair_strided(xmd[:, :K], xmd[:, K:], to_dev(W0), to_dev(W1), out0=o0, out1=o1)
    torch.cuda.synchronize()
    assert torch.all(big[:, N:N + 7] == -3.0) and torch.all(big[:, 2 * N + 7:] == -3.0)
    check(o0.contiguous(), np.ascontiguousarray(xm[:, :K]), W0, label="guard y0")
    check(o1.contiguous(), np.ascontiguousarray(xm[:, K:]), W1, label="guard y1")
    # K == 0 into strided outputs: zeros in the N columns only
    e = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    ew = torch.empty((N, 0), dtype=torch.bfloat16, device="cuda")
    big.fill_(-3.0)
    skg.gemm_pair_strided(e, e, ew, ew, out0=o0, out1=o1)
    torch.cuda.synchronize()
    assert torch.all(o0.view(torch.int16) == 0) and torch.all(o1.view(torch.int16) == 0)
    assert torch.all(big[:, N:N + 7] == -3.0) and torch.all(big[:, 2 * N + 7:] == -3.0)


def test_output_span_limits(skg):
    """The kernels store all M output rows through one buffer resource, so the span
    ((M - 1) * ldy + N) * 2 bytes must stay below 2^31. Just below it (rows 2^30 - N - 1
    elements apart) the fast kernels write near the top of the range; just above it
    (2^30 apart) the tuned plan is refused and the default call takes the
    element-wise path. Both must leave the columns between the outputs untouched."""
    M, N, K = 2, 300, 128
    free, _ = torch.cuda.mem_get_info()
    if free < 8 * 2 ** 30:
        pytest.skip("not enough device memory")
    xm, W0, W1 = _merged_case(M, N, K, seed=140)
    xmd, W0d, W1d = to_dev(xm), to_dev(W0), to_dev(W1)
    x0 = np.ascontiguousarray(xm[:, :K])
    x1 = np.ascontiguousarray(xm[:, K:])
    plan, tuned = skg.skinny_gemm_get_plan(N, K, M)
    buf = torch.empty((1 << 30) + 4 * N, dtype=torch.bfloat16, device="cuda")
    for ldy, fast in (((1 << 30) - N - 1, True), (1 << 30, False)):
        buf[:4 * N].fill_(-3.0)
        buf[ldy:ldy + 4 * N].fill_(-3.0)
        o0 = torch.as_strided(buf, (M, N), (ldy, 1), 0)
        o1 = torch.as_strided(buf, (M, N), (ldy, 1), 2 * N)
        if fast:
            skg.gemm_pair_strided(xmd[:, :K], xmd[:, K:], W0d, W1d, out0=o0, out1=o1, plan=plan)
        else:
            with pytest.raises(skg.SkinnyError) as e:
                skg.gemm_pair_strided(xmd[:, :K], xmd[:, K:], W0d, W1d, out0=o0, out1=o1, plan=plan)
            assert e.value.status == skg.SKINNY_ERR_UNSUPPORTED
            skg.gemm_pair_strided(xmd[:, :K], xmd[:, K:], W0d, W1d, out0=o0, out1=o1)
        torch.cuda.synchronize()
        check(o0.contiguous(), x0, W0, label=f"span y0 ldy={ldy}")
        check(o1.contiguous(), x1, W1, label=f"span y1 ldy={ldy}")
        for base in (0, ldy):
            assert torch.all(buf[base + N:base + 2 * N] == -3.0)
            assert torch.all(buf[base + 3 * N:base + 4 * N] == -3.0)
    del buf
    torch.cuda.empty_cache()


OFF_TABLE = [(14336, 4096), (4096, 14336), (6144, 4096), (5120, 5120), (2048, 2048), (1024, 8192),
             (3000, 1536), (100000, 4096)]


@pytest.mark.parametrize("N,K", OFF_TABLE, ids=lambda v: str(v))
def test_default_plans_off_table_full(skg, N, K):
    """Shapes the table does not hold run the default plan (the nearest tuned N's plan,
    or looped-K for an untuned K) at full size, every M, whole outputs."""
    W = synth.weights(N, K, seed=90, shape_id=N + K)
    Wd = to_dev(W)
    for M in range(1, 9):
        plan, tuned = skg.skinny_gemm_get_plan(N, K, M)
        assert not tuned
        x = synth.activations(M, K, seed=90, shape_id=N + K, tensor_id=M)
        y = skg.gemm(to_dev(x), Wd)
        torch.cuda.synchronize()
        check(y, x, W, label=f"default ({N},{K}) M={M} {plan}")
