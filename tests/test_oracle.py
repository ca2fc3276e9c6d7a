"""Pins for the CPU oracle (no GPU).

The oracle (oracle/skinny_oracle.c) is checked here against things other than
itself: hand-derived closed-form rounding cases, exact rational arithmetic with
integer rounding (tests/exact_ref.py), torch's own float32->bfloat16 conversion,
numpy's float64 matrix product, and special inputs whose product is known in
closed form (zero, identity, one-hot, small integers, power-of-two scaling).
Each is chosen so that a plausible slip (a dropped term, a wrong index, a
transposed operand, truncation instead of rounding, double rounding through
float32, a lost sign) fails at least one of them.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import synth
from tests import exact_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64_of_bits(bits):
    with np.errstate(invalid="ignore"):
        return synth.bf16_bits_to_f32(bits).astype(np.float64)


# ----------------------------------------------------------------------------
# bfloat16 <-> double helpers
# ----------------------------------------------------------------------------

def test_golden_rounding_cases(oracle_mod):
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rounding_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((float.fromhex(parts[0]), int(parts[1], 16), " ".join(parts[2:])))
    assert len(rows) >= 20
    vals = np.array([r[0] for r in rows], dtype=np.float64)
    got = oracle_mod.f64_to_bf16(vals)
    for (v, want, note), g in zip(rows, got):
        assert int(g) == want, f"{v!r} ({note}): got 0x{int(g):04X}, want 0x{want:04X}"


def test_nan_and_inf(oracle_mod):
    out = oracle_mod.f64_to_bf16(np.array([np.nan, -np.nan, np.inf, -np.inf]))
    assert (out[0] & 0x7F80) == 0x7F80 and (out[0] & 0x7F) != 0  # NaN stays NaN
    assert (out[1] & 0x7F80) == 0x7F80 and (out[1] & 0x7F) != 0
    assert (out[0] & 0x0040) and (out[1] & 0x0040)  # quiet
    assert out[2] == 0x7F80 and out[3] == 0xFF80


def test_exhaustive_roundtrip(oracle_mod):
    """All 65536 bfloat16 patterns widen exactly and round back to themselves."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    d = oracle_mod.bf16_to_f64(bits)
    # widening matches numpy's float32 view of the same top-half bits
    np.testing.assert_array_equal(d[~np.isnan(d)], _f64_of_bits(bits)[~np.isnan(d)])
    back = oracle_mod.f64_to_bf16(d)
    nan = np.isnan(d)
    np.testing.assert_array_equal(back[~nan], bits[~nan])
    assert np.all((back[nan] & 0x7F80) == 0x7F80) and np.all((back[nan] & 0x7F) != 0)


def test_exhaustive_midpoints(oracle_mod):
    """Every midpoint between consecutive finite bfloat16 values goes to the even
    neighbour; one double ulp either side goes to the nearer neighbour."""
    pos = np.arange(0x0000, 0x7F7F, dtype=np.uint16)  # a, with successor a+1 finite
    lo = _f64_of_bits(pos)
    hi = _f64_of_bits(pos + 1)
    mid = (lo + hi) / 2.0  # exact in double
    for sign in (1.0, -1.0):
        sbit = np.uint16(0x8000) if sign < 0 else np.uint16(0)
        got_mid = oracle_mod.f64_to_bf16(sign * mid)
        even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
        np.testing.assert_array_equal(got_mid, even | sbit)
        below = oracle_mod.f64_to_bf16(sign * np.nextafter(mid, 0.0))
        np.testing.assert_array_equal(below, pos | sbit)
        above = oracle_mod.f64_to_bf16(sign * np.nextafter(mid, np.inf))
        np.testing.assert_array_equal(above, (pos + 1).astype(np.uint16) | sbit)


def test_rounding_matches_torch_for_float32_inputs(oracle_mod):
    """For values that are exact float32 numbers, one double->bf16 rounding must
    agree with torch's float32->bfloat16 (round to nearest even)."""
    g = np.random.default_rng(1234)
    u = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # stay clear of float32 values that round past the bfloat16 range (torch gives inf too,
    # but keep the comparison on the finite part of the format)
    ref = synth.f32_to_bf16_bits(f)
    got = oracle_mod.f64_to_bf16(f.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_no_double_rounding(oracle_mod):
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(v) == np.float32(1.0 + 2.0 ** -8)  # a float32 detour lands on the tie
    assert int(oracle_mod.f64_to_bf16(np.array([v]))[0]) == 0x3F81


def test_rounding_against_exact_integer_route(oracle_mod):
    """Random doubles of every binade: oracle rounding == exact rational rounding."""
    from fractions import Fraction

    g = np.random.default_rng(99)
    mant = g.random(3000) + 1.0
    exps = g.integers(-140, 129, size=3000)
    vals = np.ldexp(mant, exps) * np.where(g.random(3000) < 0.5, -1.0, 1.0)
    got = oracle_mod.f64_to_bf16(vals)
    for v, gbits in zip(vals, got):
        want = exact_ref.fraction_to_bf16(Fraction(float(v)))
        assert int(gbits) == want, (v, hex(int(gbits)), hex(want))


# ----------------------------------------------------------------------------
# The product itself
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(200))
def test_brute_force_fraction(oracle_mod, seed):
    """Exact rational sums, exactly rounded, must equal the oracle bit for bit."""
    g = np.random.default_rng([7, seed])
    M = int(g.integers(1, 9))
    N = int(g.integers(1, 9))
    K = int(g.integers(1, 33))
    x = synth.normal_bf16((M, K), 1.0, g)
    W = synth.normal_bf16((N, K), 1.0 / np.sqrt(K), g)
    y, ref64, mag = oracle_mod.gemm(x, W, nthreads=1 + seed % 3)
    want, sums = exact_ref.exact_gemm(x.tolist(), W.tolist())
    np.testing.assert_array_equal(y, np.array(want, dtype=np.uint16))
    for m in range(M):
        for n in range(N):
            # double accumulation of at most 32 exact products is exact or within 1 ulp
            assert abs(ref64[m, n] - float(sums[m][n])) <= 1e-15 * max(1.0, mag[m, n])


def test_numpy_float64_blas(oracle_mod):
    """Config-shaped inputs: ref64 agrees with numpy's float64 product, y with its rounding."""
    for (N, K, M) in [(256, 1024, 1), (128, 4096, 4), (192, 1536, 2), (64, 128, 3), (96, 4096, 8)]:
        x = synth.activations(M, K, seed=0, shape_id=N, tensor_id=0)
        W = synth.weights(N, K, seed=0, shape_id=N, tensor_id=1)
        y, ref64, mag = oracle_mod.gemm(x, W)
        x64 = _f64_of_bits(x)
        W64 = _f64_of_bits(W)
        ref_np = x64 @ W64.T
        assert np.all(np.abs(ref64 - ref_np) <= 1e-12 * mag + 1e-300)
        # mag is the sum of absolute products
        np.testing.assert_allclose(mag, np.abs(x64) @ np.abs(W64).T, rtol=1e-12, atol=0)
        # rounding numpy's result the same way changes nothing except at a proven tie,
        # which needs the two doubles to straddle a midpoint; none occur here
        y_np = oracle_mod.f64_to_bf16(ref_np)
        np.testing.assert_array_equal(y, y_np)


def test_not_transposed(oracle_mod):
    """A non-square case where x.W (wrong orientation) is not even defined the same way."""
    g = np.random.default_rng(5)
    x = synth.small_int_bf16((2, 3), -3, 3, g)
    W = synth.small_int_bf16((5, 3), -3, 3, g)
    y, ref64, _ = oracle_mod.gemm(x, W)
    xi = _f64_of_bits(x)
    Wi = _f64_of_bits(W)
    for m in range(2):
        for n in range(5):
            assert ref64[m, n] == sum(xi[m, k] * Wi[n, k] for k in range(3))
    assert y.shape == (2, 5)


def test_zero_weight(oracle_mod):
    x = synth.activations(4, 256, seed=3)
    W = np.zeros((37, 256), dtype=np.uint16)
    y, ref64, mag = oracle_mod.gemm(x, W)
    assert np.all(y == 0) and np.all(ref64 == 0) and np.all(mag == 0)


def test_identity_weight(oracle_mod):
    K = 300
    x = synth.activations(3, K, seed=4)
    W = np.zeros((K, K), dtype=np.uint16)
    W[np.arange(K), np.arange(K)] = synth.BF16_ONE
    y, _, _ = oracle_mod.gemm(x, W)
    np.testing.assert_array_equal(y, x)


def test_one_hot_rows(oracle_mod):
    """W[n, pi(n)] = 1  ->  y[m, n] = x[m, pi(n)] exactly."""
    K, N = 512, 200
    g = np.random.default_rng(8)
    perm = g.integers(0, K, size=N)
    x = synth.activations(4, K, seed=5)
    W = np.zeros((N, K), dtype=np.uint16)
    W[np.arange(N), perm] = synth.BF16_ONE
    y, _, _ = oracle_mod.gemm(x, W)
    np.testing.assert_array_equal(y, x[:, perm])


def test_one_hot_activation(oracle_mod):
    """x = e_j  ->  y[:, n] = W[n, j] exactly."""
    K, N = 640, 90
    W = synth.weights(N, K, seed=6)
    for j in (0, 1, 319, K - 1):
        x = np.zeros((2, K), dtype=np.uint16)
        x[:, j] = synth.BF16_ONE
        y, _, _ = oracle_mod.gemm(x, W)
        np.testing.assert_array_equal(y[0], W[:, j])
        np.testing.assert_array_equal(y[1], W[:, j])


def test_small_integers_exact(oracle_mod):
    """Integer inputs with |sum| <= 256 give exact integer outputs."""
    g = np.random.default_rng(9)
    K = 64
    x = synth.small_int_bf16((4, K), -2, 2, g)
    W = synth.small_int_bf16((50, K), -1, 1, g)
    y, ref64, _ = oracle_mod.gemm(x, W)
    xi = np.rint(_f64_of_bits(x)).astype(np.int64)
    Wi = np.rint(_f64_of_bits(W)).astype(np.int64)
    exact = xi @ Wi.T
    assert np.all(np.abs(exact) <= 256)
    np.testing.assert_array_equal(ref64, exact.astype(np.float64))
    np.testing.assert_array_equal(_f64_of_bits(y), exact.astype(np.float64))


def test_power_of_two_scaling(oracle_mod):
    """y(2^s x) == 2^s y(x), bit for bit, away from the format's range ends."""
    x = synth.activations(2, 1024, seed=10)
    W = synth.weights(64, 1024, seed=10)
    y0, _, _ = oracle_mod.gemm(x, W)
    for s in (-8, -3, 5, 8):
        xs = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(2.0 ** s))
        ys, _, _ = oracle_mod.gemm(xs, W)
        np.testing.assert_array_equal(_f64_of_bits(ys), _f64_of_bits(y0) * 2.0 ** s)


def test_rows_independent(oracle_mod):
    """M = 8 equals eight M = 1 runs; selected rows equal the full product's columns."""
    x = synth.activations(8, 1536, seed=11)
    W = synth.weights(96, 1536, seed=11)
    y4, r4, m4 = oracle_mod.gemm(x, W)
    for m in range(8):
        y1, r1, m1 = oracle_mod.gemm(x[m:m + 1], W)
        np.testing.assert_array_equal(y1[0], y4[m])
        np.testing.assert_array_equal(r1[0], r4[m])
    rows = np.array([95, 0, 17, 17, 50], dtype=np.int64)
    ys, rs, ms = oracle_mod.gemm_rows(x, W, rows)
    np.testing.assert_array_equal(ys, y4[:, rows])
    np.testing.assert_array_equal(rs, r4[:, rows])
    np.testing.assert_array_equal(ms, m4[:, rows])


def test_thread_count_invariant(oracle_mod):
    x = synth.activations(3, 512, seed=12)
    W = synth.weights(333, 512, seed=12)
    ref = oracle_mod.gemm(x, W, nthreads=1)
    for nt in (2, 7, 64):
        out = oracle_mod.gemm(x, W, nthreads=nt)
        for a, b in zip(ref, out):
            np.testing.assert_array_equal(a, b)


def test_pair_is_two_singles(oracle_mod):
    x = synth.activations(2, 128, seed=13)
    W0 = synth.weights(64, 128, seed=13, tensor_id=1)
    W1 = synth.weights(64, 128, seed=13, tensor_id=2)
    (a0, _, _), (a1, _, _) = oracle_mod.gemm_pair(x, W0, W1)
    np.testing.assert_array_equal(a0, oracle_mod.gemm(x, W0)[0])
    np.testing.assert_array_equal(a1, oracle_mod.gemm(x, W1)[0])
    assert not np.array_equal(a0, a1)


def test_empty_shapes(oracle_mod):
    x = np.zeros((2, 0), dtype=np.uint16)
    W = np.zeros((5, 0), dtype=np.uint16)
    y, ref64, mag = oracle_mod.gemm(x, W)  # K = 0: empty sums are +0
    assert y.shape == (2, 5) and np.all(y == 0) and np.all(ref64 == 0)
    y, _, _ = oracle_mod.gemm(np.zeros((1, 4), np.uint16), np.zeros((0, 4), np.uint16))
    assert y.shape == (1, 0)


def test_f32_output_form(oracle_mod):
    """The float32-output oracle: the same double sum, rounded once to float32."""
    def b(v):
        return synth.f32_to_bf16_bits(np.array(v, np.float32))
    # exact double sums 1 + 2^-24 (float32 tie -> 1.0) and 1 + 3*2^-24 (tie -> 1 + 2^-22)
    x = np.zeros((2, 3), np.uint16)
    x[0] = b([1.0, 2.0 ** -12, 0.0])
    x[1] = b([1.0, 2.0 ** -12, 2.0 ** -11])
    W = np.zeros((1, 3), np.uint16)
    W[0] = b([1.0, 2.0 ** -12, 2.0 ** -12])
    y32, ref64, _ = oracle_mod.gemm_f32out(x, W)
    assert ref64[0, 0] == 1.0 + 2.0 ** -24 and ref64[1, 0] == 1.0 + 3 * 2.0 ** -24
    assert y32.dtype == np.float32
    assert y32[0, 0] == np.float32(1.0)
    assert y32[1, 0] == np.float32(1.0 + 2.0 ** -22)
    # just above a tie goes up (1 + 2^-24 + 2^-40 is exact in double)
    x2 = np.zeros((1, 4), np.uint16)
    x2[0] = b([1.0, 2.0 ** -12, 2.0 ** -20, 0.0])
    W2 = np.zeros((1, 4), np.uint16)
    W2[0] = b([1.0, 2.0 ** -12, 2.0 ** -20, 0.0])
    y32b, _, _ = oracle_mod.gemm_f32out(x2, W2)
    assert y32b[0, 0] == np.float32(1.0 + 2.0 ** -23)
    # small-integer products: exact
    g = np.random.default_rng(21)
    xi = synth.small_int_bf16((3, 40), -3, 3, g)
    Wi = synth.small_int_bf16((17, 40), -3, 3, g)
    y32, ref64, _ = oracle_mod.gemm_f32out(xi, Wi)
    exact = np.rint(_f64_of_bits(xi)).astype(np.int64) @ np.rint(_f64_of_bits(Wi)).astype(np.int64).T
    np.testing.assert_array_equal(y32, exact.astype(np.float32))
    # the bf16 output is the same sum rounded differently
    ybf, _, _ = oracle_mod.gemm(xi, Wi)
    np.testing.assert_array_equal(_f64_of_bits(ybf), exact.astype(np.float64))
    # selected rows
    rows = np.array([3, 0, 16], np.int64)
    y32r, _, _ = oracle_mod.gemm_f32out(xi, Wi, rows)
    np.testing.assert_array_equal(y32r, y32[:, rows])


# ----------------------------------------------------------------------------
# Acceptance rules
# ----------------------------------------------------------------------------

def test_acceptance_rules(oracle_mod):
    from oracle import accept

    x = synth.activations(2, 1024, seed=14)
    W = synth.weights(128, 1024, seed=14)
    y, ref64, mag = oracle_mod.gemm(x, W)
    r = accept.acceptance(y, y, ref64, mag)
    assert r["pass"] and r["min_cos"] == pytest.approx(1.0)
    # one element off by one bf16 ulp still passes G1/G2 (and S1 for |y| ~ 1 values)
    y2 = y.copy()
    y2[0, 5] ^= 1
    assert accept.acceptance(y2, y, ref64, mag)["g1_pass"]
    # a wrong sign on one element fails S1 and G1 (|2y| > 1e-2 * mag for these sizes)
    y3 = y.copy()
    big = int(np.argmax(np.abs(ref64[1])))
    y3[1, big] ^= 0x8000
    r3 = accept.acceptance(y3, y, ref64, mag)
    assert not r3["s1_pass"] and not r3["g1_pass"] and not r3["pass"]
    # a zero row against a non-zero row fails G2
    y4 = y.copy()
    y4[0, :] = 0
    assert not accept.acceptance(y4, y, ref64, mag)["g2_pass"]
    # float32 outputs are compared as values
    y32, _, _ = oracle_mod.gemm_f32out(x, W)
    r32 = accept.acceptance(y32, y32, ref64, mag)
    assert r32["pass"] and r32["n_bitwise_equal"] == y32.size
    y32b = y32.copy()
    y32b[1, 3] = -y32b[1, 3] - 1.0
    assert not accept.acceptance(y32b, y32, ref64, mag)["pass"]
