"""Acceptance rules for comparing a GPU result with the oracle (test infrastructure).

G1 (per element, gate):   |y - y_ref| <= 1e-2 * mag + 1e-6,
    with y_ref the oracle's bf16 output and mag = sum_k |x[m,k] * W[n,k]|.
G2 (per output row, gate): cosine(y[m, :], y_ref[m, :]) >= 0.99999 in float64;
    two all-zero rows agree, exactly one all-zero row disagrees.
S1 (per element, strict):  |y - ref64| <= 7.5e-5 + 2**-8 * |ref64|, the float64
    comparison rule of vLLM PR #65306 (SM90 skinny GEMM plans), section
    Validation.

G1 and G2 are the bar the HIP path must meet; S1 is the cited pull request's
own, tighter rule, and the parity tests assert it as well.
"""
from __future__ import annotations

import numpy as np

G1_REL = 1e-2
G1_ABS = 1e-6
G2_MIN_COS = 0.99999
S1_ABS = 7.5e-5
S1_REL = 2.0 ** -8


def _f64(vals) -> np.ndarray:
    """bfloat16 bit patterns (uint16) or float32 values -> float64."""
    a = np.asarray(vals)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    b = np.ascontiguousarray(a, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _n_bitwise_equal(a, b) -> int:
    """Number of elements whose bit patterns agree (bf16 bits or float32 values)."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.astype(np.float32).view(np.uint32)
    return int(np.sum(a == b))


def cosine_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Row-wise cosine of two float64 [R, L] arrays with the zero-row convention."""
    a = np.atleast_2d(a)
    b = np.atleast_2d(b)
    na = np.linalg.norm(a, axis=1)
    nb = np.linalg.norm(b, axis=1)
    out = np.empty(a.shape[0], dtype=np.float64)
    for i in range(a.shape[0]):
        if na[i] == 0.0 and nb[i] == 0.0:
            out[i] = 1.0
        elif na[i] == 0.0 or nb[i] == 0.0:
            out[i] = 0.0
        else:
            out[i] = float(np.dot(a[i], b[i]) / (na[i] * nb[i]))
    return out


def acceptance(y_bits, y_ref_bits, ref64, mag, check_cosine: bool = True) -> dict:
    """Evaluate G1, G2 and S1 for one [M, L] output block.

    y_bits / y_ref_bits are bfloat16 bit patterns (uint16), or float32 values for
    the float32-output form (both arrays of the same kind).

    Returns a dict with the pass flags and the worst margins: max_g1_ratio and
    max_s1_ratio are max(|err| / bound) (<= 1 passes), min_cos the smallest row
    cosine. Set check_cosine=False when the block is a sample of columns rather
    than whole rows.
    """
    y = _f64(y_bits)
    yr = _f64(y_ref_bits)
    ref64 = np.asarray(ref64, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    finite = np.isfinite(y)
    err_g1 = np.abs(y - yr)
    bound_g1 = G1_REL * mag + G1_ABS
    err_s1 = np.abs(y - ref64)
    bound_s1 = S1_ABS + S1_REL * np.abs(ref64)
    with np.errstate(invalid="ignore"):
        g1_ok = bool(np.all(finite) and np.all(err_g1 <= bound_g1))
        s1_ok = bool(np.all(finite) and np.all(err_s1 <= bound_s1))
        g1_ratio = float(np.max(err_g1 / bound_g1)) if y.size else 0.0
        s1_ratio = float(np.max(err_s1 / bound_s1)) if y.size else 0.0
    res = {
        "g1_pass": g1_ok,
        "s1_pass": s1_ok,
        "max_g1_ratio": g1_ratio,
        "max_s1_ratio": s1_ratio,
        "max_abs_err": float(np.max(err_g1)) if y.size else 0.0,
        "n_bitwise_equal": _n_bitwise_equal(y_bits, y_ref_bits),
        "n": int(y.size),
    }
    if check_cosine:
        cos = cosine_rows(y.reshape(y.shape[0], -1) if y.ndim > 1 else y[None],
                          yr.reshape(yr.shape[0], -1) if yr.ndim > 1 else yr[None])
        res["min_cos"] = float(cos.min()) if cos.size else 1.0
        res["g2_pass"] = bool(np.all(cos >= G2_MIN_COS))
    else:
        res["min_cos"] = None
        res["g2_pass"] = True
    res["pass"] = res["g1_pass"] and res["g2_pass"] and res["s1_pass"]
    return res
