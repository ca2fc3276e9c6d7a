"""Exact rational reference used to pin the oracle (tests only).

The sum of products is formed exactly with ``fractions.Fraction`` and rounded to
bfloat16 by integer arithmetic: the value is scaled by the spacing of bfloat16
numbers in its binade, split into integer part and remainder, and the remainder
is compared with one half (ties go to the even integer). This shares no step
with the oracle's double-precision ``rint`` route, so a mistake in either shows
up as a mismatch.
"""
from __future__ import annotations

import struct
from fractions import Fraction

BF16_MAX = Fraction(255) * Fraction(2) ** 120  # (2 - 2^-7) * 2^127


def bf16_to_fraction(bits: int) -> Fraction:
    """Exact value of a finite bfloat16 bit pattern, by its fields."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("not finite")
    if exp == 0:
        val = Fraction(man) * Fraction(2) ** (-133)          # subnormal: man * 2^-126 * 2^-7
    else:
        val = Fraction(128 + man) * Fraction(2) ** (exp - 127 - 7)
    return sign * val


def _floor_log2(v: Fraction) -> int:
    """floor(log2(v)) for v > 0, exactly."""
    n, d = v.numerator, v.denominator
    e = n.bit_length() - d.bit_length()
    # now 2^(e-1) < n/d < 2^(e+1); adjust to the exact floor
    if Fraction(2) ** e > v:
        e -= 1
    return e


def fraction_to_bf16(v: Fraction) -> int:
    """Round an exact rational to bfloat16, nearest with ties to even."""
    if v == 0:
        return 0x0000
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    e = max(_floor_log2(a), -126)
    q = Fraction(2) ** (e - 7)
    t = a / q
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * q
    if r > BF16_MAX:
        return sign | 0x7F80
    # encode r exactly: normal if r >= 2^-126, else subnormal
    if r == 0:
        return sign
    if r >= Fraction(2) ** -126:
        e2 = _floor_log2(r)
        man = r / Fraction(2) ** (e2 - 7) - 128
        assert man.denominator == 1 and 0 <= man < 128
        return sign | ((e2 + 127) << 7) | int(man)
    man = r / Fraction(2) ** (-133)
    assert man.denominator == 1 and 0 < man < 128
    return sign | int(man)


def exact_gemm(x_bits, W_bits):
    """Exact y = bf16(x . W^T) for small integer-bit lists: returns (y_bits, exact sums)."""
    M = len(x_bits)
    N = len(W_bits)
    xf = [[bf16_to_fraction(int(b)) for b in row] for row in x_bits]
    wf = [[bf16_to_fraction(int(b)) for b in row] for row in W_bits]
    y = [[0] * N for _ in range(M)]
    s = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for a, b in zip(xf[m], wf[n]):
                acc += a * b
            s[m][n] = acc
            y[m][n] = fraction_to_bf16(acc)
    return y, s


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]
