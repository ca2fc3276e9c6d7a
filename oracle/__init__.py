"""Python face of the CPU oracle for the BF16 skinny GEMM.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, never by the HIP library or its
binding. It loads ``oracle/libskinny_oracle.so`` (plain C, see
``skinny_oracle.c`` for the definition and its sources) and marshals numpy
arrays of bfloat16 bit patterns (uint16) into it.

Every function here is pinned by ``tests/test_oracle.py`` against exact rational
arithmetic, closed forms, special cases and numpy's float64 BLAS; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .accept import acceptance, cosine_rows  # noqa: F401  (re-export)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "skinny_oracle.c")
LIB_PATH = os.path.join(_HERE, "libskinny_oracle.so")

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE double semantics, no contraction)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_bf16_to_f64_array.restype = None
        lib.oracle_bf16_to_f64_array.argtypes = [u16p, f64p, ctypes.c_size_t]
        lib.oracle_f64_to_bf16_array.restype = None
        lib.oracle_f64_to_bf16_array.argtypes = [f64p, u16p, ctypes.c_size_t]
        lib.oracle_gemm_bf16_rows.restype = ctypes.c_int
        lib.oracle_gemm_bf16_rows.argtypes = [u16p, u16p, i64p, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, u16p, f64p, f64p, f64p, ctypes.c_int]
        _lib = lib
        return lib


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    """Host threads the oracle uses by default: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_bf16_to_f64_array(_p(b, ctypes.c_uint16), _p(out, ctypes.c_double), b.size)
    return out


def f64_to_bf16(values) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, one round-to-nearest-even step."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_f64_to_bf16_array(_p(v, ctypes.c_double), _p(out, ctypes.c_uint16), v.size)
    return out


def gemm_rows(x_bits, W_bits, rows=None, nthreads: int | None = None):
    """Oracle for selected output columns n (rows of W).

    x_bits: uint16 [M, K]; W_bits: uint16 [N, K] (any N; only `rows` are read);
    rows: int64 indices into W, or None for all rows.
    Returns (y_bits [M, R], ref64 [M, R], mag [M, R]) with R = len(rows).
    """
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W = np.ascontiguousarray(W_bits, dtype=np.uint16) if not isinstance(W_bits, np.memmap) else W_bits
    if x.ndim != 2 or W.ndim != 2 or x.shape[1] != W.shape[1]:
        raise ValueError(f"shape mismatch: x {x.shape}, W {W.shape}")
    M, K = x.shape
    if rows is None:
        r = None
        nrows = W.shape[0]
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        if r.size and (r.min() < 0 or r.max() >= W.shape[0]):
            raise ValueError("row index out of range")
        nrows = r.size
    y = np.empty((M, nrows), dtype=np.uint16)
    ref = np.empty((M, nrows), dtype=np.float64)
    mag = np.empty((M, nrows), dtype=np.float64)
    x64 = np.empty((M, K), dtype=np.float64)
    nt = default_threads() if nthreads is None else int(nthreads)
    rc = _load().oracle_gemm_bf16_rows(
        _p(x, ctypes.c_uint16), _p(W, ctypes.c_uint16),
        _p(r, ctypes.c_int64) if r is not None else None, nrows, M, K,
        _p(y, ctypes.c_uint16), _p(ref, ctypes.c_double), _p(mag, ctypes.c_double),
        _p(x64, ctypes.c_double), nt)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_bf16_rows failed ({rc})")
    return y, ref, mag


def gemm(x_bits, W_bits, nthreads: int | None = None):
    """Oracle for the full product y = x . W^T: (y_bits [M,N], ref64, mag)."""
    return gemm_rows(x_bits, W_bits, None, nthreads)


def gemm_f32out(x_bits, W_bits, rows=None, nthreads: int | None = None):
    """Oracle for the float32-output form: the same float64 sum, rounded once to
    float32 (IEEE round-to-nearest-even, numpy's float64 -> float32 conversion).
    Returns (y32 [M, R] float32, ref64, mag)."""
    _, ref64, mag = gemm_rows(x_bits, W_bits, rows, nthreads)
    return ref64.astype(np.float32), ref64, mag


def gemm_pair(x_bits, W0_bits, W1_bits, nthreads: int | None = None):
    """Paired form: the same definition applied to W0 and to W1 with one shared x."""
    return gemm(x_bits, W0_bits, nthreads), gemm(x_bits, W1_bits, nthreads)
