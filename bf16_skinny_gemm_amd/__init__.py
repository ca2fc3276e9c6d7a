"""BF16 skinny GEMM for MI355X (gfx950): y[M,N] = x[M,K] . W[N,K]^T for M = 1..8.

Thin Python binding over the C ABI of ``libskinny_gemm_bf16.so``
(``include/skinny_gemm.h``). Every step of the computation runs in the HIP
kernels; this module only marshals arguments. PyTorch provides device memory
and the current stream. There is no fallback: if the library is missing, or the
device is not gfx950, calls raise.

Raw entry points (same names and arguments as the C functions; pointers as
Python ints; a non-zero status raises :class:`SkinnyError`):
    skinny_gemm_init, skinny_gemm_bf16, skinny_gemm_bf16_pair,
    skinny_gemm_bf16_ex, skinny_gemm_bf16_pair_ex, skinny_gemm_bf16_pair_strided,
    skinny_gemm_bf16_pair_strided_ex, skinny_gemm_bf16_f32out,
    skinny_gemm_bf16_f32out_ex, skinny_gemm_get_plan,
    skinny_gemm_num_variants, skinny_gemm_get_variant,
    skinny_gemm_status_string, skinny_gemm_version,
    skinny_gemm_split_k_workspace_bytes, skinny_gemm_bf16_split_k,
    skinny_gemm_bf16_split_k_noalloc, skinny_gemm_split_k_num_variants,
    skinny_gemm_split_k_get_variant, skinny_gemm_split_k_default_plan

Tensor helpers: :func:`gemm`, :func:`gemm_pair`, :func:`gemm_pair_strided`,
:func:`split_k_workspace`, :func:`gemm_split_k` and :func:`gemm_split_k_noalloc`.
"""
from __future__ import annotations

import ctypes
import os
import threading

# torch first: its HIP runtime (soname libamdhip64.so.7) must be the one the
# library binds to, so that torch's stream handles are valid in it.
import torch

from .build import LIB_PATH

SKINNY_OK = 0
SKINNY_ERR_INVALID_ARG = -1
SKINNY_ERR_UNSUPPORTED = -2
SKINNY_ERR_NOT_INITIALIZED = -3
SKINNY_ERR_LAUNCH = -4

SKINNY_KIND_FIXED_K = 1
SKINNY_KIND_LOOP_K = 2
SKINNY_KIND_SCALAR = 3
SKINNY_KIND_MFMA = 4
SKINNY_KIND_SPLIT_K = 5


class SkinnyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_status_string(status)} (status {status})")


class Plan(ctypes.Structure):
    """skinny_plan_t."""

    _fields_ = [
        ("kind", ctypes.c_int32),
        ("threads_per_block", ctypes.c_int32),
        ("lanes_per_row", ctypes.c_int32),
        ("chunks", ctypes.c_int32),
        ("rows_per_wave", ctypes.c_int32),
        ("k_split", ctypes.c_int32),
        ("nontemporal", ctypes.c_int32),
        ("grid_blocks", ctypes.c_int32),
        ("x_in_lds", ctypes.c_int32),
        ("prefetch", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f, _ in self._fields_}

    @classmethod
    def from_dict(cls, d: dict) -> "Plan":
        return cls(**{f: int(d[f]) for f, _ in cls._fields_})

    def __repr__(self) -> str:
        return "Plan(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first (python -m bf16_skinny_gemm_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        i = ctypes.c_int
        pp = ctypes.POINTER(Plan)
        L.skinny_gemm_init.argtypes = [i]
        L.skinny_gemm_bf16.argtypes = [vp, vp, vp, i, i, i, vp]
        L.skinny_gemm_bf16_pair.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp]
        L.skinny_gemm_bf16_ex.argtypes = [vp, vp, vp, i, i, i, pp, vp]
        L.skinny_gemm_bf16_pair_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, pp, vp]
        L.skinny_gemm_bf16_f32out.argtypes = [vp, vp, vp, i, i, i, vp]
        L.skinny_gemm_bf16_pair_strided.argtypes = [vp, vp, i, vp, vp, vp, vp, i, i, i, i, vp]
        L.skinny_gemm_bf16_pair_strided_ex.argtypes = [vp, vp, i, vp, vp, vp, vp, i, i, i, i, pp, vp]
        L.skinny_gemm_bf16_f32out_ex.argtypes = [vp, vp, vp, i, i, i, pp, vp]
        L.skinny_gemm_get_plan.argtypes = [i, i, i, pp]
        L.skinny_gemm_num_variants.argtypes = []
        L.skinny_gemm_get_variant.argtypes = [i, pp]
        L.skinny_gemm_status_string.argtypes = [i]
        L.skinny_gemm_status_string.restype = ctypes.c_char_p
        L.skinny_gemm_version.argtypes = []
        L.skinny_gemm_split_k_workspace_bytes.argtypes = [i, i, i, pp]
        L.skinny_gemm_split_k_workspace_bytes.restype = ctypes.c_size_t
        L.skinny_gemm_bf16_split_k.argtypes = [vp, vp, vp, i, i, i, pp, vp, ctypes.c_size_t, vp]
        L.skinny_gemm_bf16_split_k_noalloc.argtypes = [vp, vp, vp, i, i, i, pp, vp]
        L.skinny_gemm_split_k_num_variants.argtypes = []
        L.skinny_gemm_split_k_get_variant.argtypes = [i, pp]
        L.skinny_gemm_split_k_default_plan.argtypes = [i, i, i, pp]
        for name in ("skinny_gemm_init", "skinny_gemm_bf16", "skinny_gemm_bf16_pair",
                     "skinny_gemm_bf16_ex", "skinny_gemm_bf16_pair_ex", "skinny_gemm_bf16_f32out",
                     "skinny_gemm_bf16_f32out_ex", "skinny_gemm_bf16_pair_strided",
                     "skinny_gemm_bf16_pair_strided_ex", "skinny_gemm_get_plan",
                     "skinny_gemm_num_variants", "skinny_gemm_get_variant", "skinny_gemm_version",
                     "skinny_gemm_bf16_split_k", "skinny_gemm_bf16_split_k_noalloc",
                     "skinny_gemm_split_k_num_variants", "skinny_gemm_split_k_get_variant",
                     "skinny_gemm_split_k_default_plan"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
        return L


def _status_string(status: int) -> str:
    try:
        return lib().skinny_gemm_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - library not loadable
        return "unknown status"


def _check(status: int, where: str) -> int:
    if status < 0:
        raise SkinnyError(status, where)
    return status


# ---- raw entry points (same names as the C ABI) -----------------------------

def skinny_gemm_init(device: int) -> None:
    _check(lib().skinny_gemm_init(int(device)), "skinny_gemm_init")


def skinny_gemm_bf16(x: int, W: int, y: int, M: int, N: int, K: int, stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16(x, W, y, M, N, K, stream), "skinny_gemm_bf16")


def skinny_gemm_bf16_pair(x: int, W0: int, W1: int, y0: int, y1: int, M: int, N: int, K: int,
                          stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_pair(x, W0, W1, y0, y1, M, N, K, stream), "skinny_gemm_bf16_pair")


def skinny_gemm_bf16_ex(x: int, W: int, y: int, M: int, N: int, K: int, plan: Plan,
                        stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_ex(x, W, y, M, N, K, ctypes.byref(plan), stream),
           "skinny_gemm_bf16_ex")


def skinny_gemm_bf16_pair_ex(x: int, W0: int, W1: int, y0: int, y1: int, M: int, N: int, K: int,
                             plan: Plan, stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_pair_ex(x, W0, W1, y0, y1, M, N, K, ctypes.byref(plan), stream),
           "skinny_gemm_bf16_pair_ex")


def skinny_gemm_bf16_pair_strided(x0: int, x1: int, ldx: int, W0: int, W1: int, y0: int, y1: int,
                                  ldy: int, M: int, N: int, K: int, stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_pair_strided(x0, x1, ldx, W0, W1, y0, y1, ldy, M, N, K, stream),
           "skinny_gemm_bf16_pair_strided")


def skinny_gemm_bf16_pair_strided_ex(x0: int, x1: int, ldx: int, W0: int, W1: int, y0: int, y1: int,
                                     ldy: int, M: int, N: int, K: int, plan: Plan,
                                     stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_pair_strided_ex(x0, x1, ldx, W0, W1, y0, y1, ldy, M, N, K,
                                                  ctypes.byref(plan), stream),
           "skinny_gemm_bf16_pair_strided_ex")


def skinny_gemm_bf16_f32out(x: int, W: int, y: int, M: int, N: int, K: int, stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_f32out(x, W, y, M, N, K, stream), "skinny_gemm_bf16_f32out")


def skinny_gemm_bf16_f32out_ex(x: int, W: int, y: int, M: int, N: int, K: int, plan: Plan,
                               stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_f32out_ex(x, W, y, M, N, K, ctypes.byref(plan), stream),
           "skinny_gemm_bf16_f32out_ex")


def skinny_gemm_get_plan(N: int, K: int, M: int) -> tuple[Plan, bool]:
    """(plan, tuned): the plan skinny_gemm_bf16 uses for (N, K, M)."""
    p = Plan()
    r = _check(lib().skinny_gemm_get_plan(N, K, M, ctypes.byref(p)), "skinny_gemm_get_plan")
    return p, bool(r == 1)


def skinny_gemm_num_variants() -> int:
    return lib().skinny_gemm_num_variants()


def skinny_gemm_get_variant(index: int) -> Plan:
    p = Plan()
    _check(lib().skinny_gemm_get_variant(index, ctypes.byref(p)), "skinny_gemm_get_variant")
    return p


def skinny_gemm_status_string(status: int) -> str:
    return _status_string(status)


def skinny_gemm_version() -> int:
    return lib().skinny_gemm_version()


def variants() -> list[Plan]:
    return [skinny_gemm_get_variant(i) for i in range(skinny_gemm_num_variants())]


def _plan_ref(plan: Plan | None):
    return ctypes.byref(plan) if plan is not None else None


def skinny_gemm_split_k_workspace_bytes(M: int, N: int, K: int, plan: Plan | None = None) -> int:
    """Workspace bytes of a split-K call (0: no call with these arguments is accepted)."""
    return int(lib().skinny_gemm_split_k_workspace_bytes(M, N, K, _plan_ref(plan)))


def skinny_gemm_bf16_split_k(x: int, W: int, y: int, M: int, N: int, K: int, plan: Plan | None,
                             workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_split_k(x, W, y, M, N, K, _plan_ref(plan), workspace,
                                          workspace_bytes, stream), "skinny_gemm_bf16_split_k")


def skinny_gemm_bf16_split_k_noalloc(x: int, W: int, y: int, M: int, N: int, K: int,
                                     plan: Plan | None = None, stream: int = 0) -> None:
    _check(lib().skinny_gemm_bf16_split_k_noalloc(x, W, y, M, N, K, _plan_ref(plan), stream),
           "skinny_gemm_bf16_split_k_noalloc")


def skinny_gemm_split_k_num_variants() -> int:
    return lib().skinny_gemm_split_k_num_variants()


def skinny_gemm_split_k_get_variant(index: int) -> Plan:
    p = Plan()
    _check(lib().skinny_gemm_split_k_get_variant(index, ctypes.byref(p)),
           "skinny_gemm_split_k_get_variant")
    return p


def skinny_gemm_split_k_default_plan(M: int, N: int, K: int) -> Plan:
    p = Plan()
    _check(lib().skinny_gemm_split_k_default_plan(M, N, K, ctypes.byref(p)),
           "skinny_gemm_split_k_default_plan")
    return p


def split_k_variants() -> list[Plan]:
    return [skinny_gemm_split_k_get_variant(i) for i in range(skinny_gemm_split_k_num_variants())]


# ---- tensor helpers ---------------------------------------------------------

_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device: torch.device) -> int:
    """The raw handle of torch's current stream on `device` (no Stream object built
    when torch exposes the raw getter)."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if _raw_stream is not None:
        return int(_raw_stream(idx))
    return int(torch.cuda.current_stream(idx).cuda_stream)


class _on_device:
    """Make `device` current for the call, switching only when it is not already."""

    __slots__ = ("idx", "prev")

    def __init__(self, device: torch.device):
        self.idx = device.index
        self.prev = None

    def __enter__(self):
        if self.idx is not None:
            cur = torch.cuda.current_device()
            if cur != self.idx:
                self.prev = cur
                torch.cuda.set_device(self.idx)
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)
        return False


def _check_tensor(t: torch.Tensor, name: str, ndim: int = 2) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def gemm(x: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None,
         plan: Plan | None = None, out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """y = x @ W.T for bfloat16 x [M, K] (M <= 8) and W [N, K]; one kernel launch
    on the current stream. out_dtype torch.float32 keeps the float32 sums
    (skinny_gemm_bf16_f32out)."""
    _check_tensor(x, "x")
    _check_tensor(W, "W")
    M, K = x.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: x {tuple(x.shape)}, W {tuple(W.shape)}")
    if W.device != x.device:
        raise ValueError("x and W must be on the same device")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out_dtype must be bfloat16 or float32, got {out_dtype}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        if out.dtype != out_dtype or out.device != x.device or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous {out_dtype} tensor on {x.device}")
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be [{M}, {N}]")
    s = _stream_handle(x.device)
    with _on_device(x.device):
        if out_dtype == torch.float32:
            if plan is None:
                skinny_gemm_bf16_f32out(x.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K, s)
            else:
                skinny_gemm_bf16_f32out_ex(x.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K,
                                           plan, s)
        elif plan is None:
            skinny_gemm_bf16(x.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K, s)
        else:
            skinny_gemm_bf16_ex(x.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K, plan, s)
    return out


def gemm_pair(x: torch.Tensor, W0: torch.Tensor, W1: torch.Tensor,
              out0: torch.Tensor | None = None, out1: torch.Tensor | None = None,
              plan: Plan | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """(x @ W0.T, x @ W1.T) for two same-shape bfloat16 weights, one kernel launch."""
    _check_tensor(x, "x")
    _check_tensor(W0, "W0")
    _check_tensor(W1, "W1")
    M, K = x.shape
    if tuple(W0.shape) != tuple(W1.shape) or W0.shape[1] != K:
        raise ValueError(f"shapes: x {tuple(x.shape)}, W0 {tuple(W0.shape)}, W1 {tuple(W1.shape)}")
    N = W0.shape[0]
    if W0.device != x.device or W1.device != x.device:
        raise ValueError("x, W0 and W1 must be on the same device")
    outs = []
    for o, name in ((out0, "out0"), (out1, "out1")):
        if o is None:
            o = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        else:
            _check_tensor(o, name)
            if o.device != x.device:
                raise ValueError(f"{name} must be on {x.device}")
            if tuple(o.shape) != (M, N):
                raise ValueError(f"{name} must be [{M}, {N}]")
        outs.append(o)
    s = _stream_handle(x.device)
    with _on_device(x.device):
        if plan is None:
            skinny_gemm_bf16_pair(x.data_ptr(), W0.data_ptr(), W1.data_ptr(), outs[0].data_ptr(),
                                  outs[1].data_ptr(), M, N, K, s)
        else:
            skinny_gemm_bf16_pair_ex(x.data_ptr(), W0.data_ptr(), W1.data_ptr(), outs[0].data_ptr(),
                                     outs[1].data_ptr(), M, N, K, plan, s)
    return outs[0], outs[1]


def _check_rowview(t: torch.Tensor, name: str) -> None:
    """A 2-D bfloat16 GPU view with unit column stride (rows may be strided)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.device.type != "cuda":
        raise TypeError(f"{name} must be a bfloat16 GPU tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride, got stride {t.stride()}")


def gemm_pair_strided(x0: torch.Tensor, x1: torch.Tensor, W0: torch.Tensor, W1: torch.Tensor,
                      out0: torch.Tensor | None = None, out1: torch.Tensor | None = None,
                      plan: Plan | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """(x0 @ W0.T, x1 @ W1.T) in one launch, x0 and x1 being row-strided views with
    the same row stride (e.g. the two halves of a merged [M, 2K] activation); out0
    and out1 may likewise be views of one merged [M, 2N] output."""
    _check_rowview(x0, "x0")
    _check_rowview(x1, "x1")
    _check_tensor(W0, "W0")
    _check_tensor(W1, "W1")
    M, K = x0.shape
    if tuple(x1.shape) != (M, K) or x1.stride(0) != x0.stride(0):
        raise ValueError("x0 and x1 must have the same shape and row stride")
    if tuple(W0.shape) != tuple(W1.shape) or W0.shape[1] != K:
        raise ValueError(f"shapes: x {tuple(x0.shape)}, W0 {tuple(W0.shape)}, W1 {tuple(W1.shape)}")
    N = W0.shape[0]
    if x1.device != x0.device or W0.device != x0.device or W1.device != x0.device:
        raise ValueError("x0, x1, W0 and W1 must be on the same device")
    if out0 is None and out1 is None:
        merged = torch.empty((M, 2 * N), dtype=torch.bfloat16, device=x0.device)
        out0, out1 = merged[:, :N], merged[:, N:]
    elif out0 is None or out1 is None:
        raise ValueError("give both out0 and out1, or neither")
    for o, name in ((out0, "out0"), (out1, "out1")):
        _check_rowview(o, name)
        if o.device != x0.device:
            raise ValueError(f"{name} must be on {x0.device}")
        if tuple(o.shape) != (M, N):
            raise ValueError(f"{name} must be [{M}, {N}]")
    if out0.stride(0) != out1.stride(0):
        raise ValueError("out0 and out1 must have the same row stride")
    ldx = x0.stride(0) if M > 1 else K
    ldy = out0.stride(0) if M > 1 else N
    s = _stream_handle(x0.device)
    with _on_device(x0.device):
        args = (x0.data_ptr(), x1.data_ptr(), ldx, W0.data_ptr(), W1.data_ptr(), out0.data_ptr(),
                out1.data_ptr(), ldy, M, N, K)
        if plan is None:
            skinny_gemm_bf16_pair_strided(*args, s)
        else:
            skinny_gemm_bf16_pair_strided_ex(*args, plan, s)
    return out0, out1


def split_k_workspace(M: int, N: int, K: int, plan: Plan | None = None,
                      device: torch.device | str = "cuda") -> torch.Tensor:
    """A zero-filled uint8 device buffer big enough for split-K calls of this shape
    and plan (allocate it once, outside any graph capture, and reuse it)."""
    nbytes = skinny_gemm_split_k_workspace_bytes(M, N, K, plan)
    if nbytes == 0:
        raise SkinnyError(SKINNY_ERR_INVALID_ARG, "skinny_gemm_split_k_workspace_bytes")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _split_args(x: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None):
    _check_tensor(x, "x")
    _check_tensor(W, "W")
    M, K = x.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: x {tuple(x.shape)}, W {tuple(W.shape)}")
    if W.device != x.device:
        raise ValueError("x and W must be on the same device")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _check_tensor(out, "out")
        if out.device != x.device or tuple(out.shape) != (M, N):
            raise ValueError(f"out must be a contiguous bfloat16 [{M}, {N}] tensor on {x.device}")
    return M, N, K, out


def gemm_split_k(x: torch.Tensor, W: torch.Tensor, workspace: torch.Tensor,
                 plan: Plan | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """y = x @ W.T with cross-block split-K (skinny_gemm_bf16_split_k), partials in
    `workspace` (from split_k_workspace, reused across calls on one stream)."""
    M, N, K, out = _split_args(x, W, out)
    if workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {x.device}")
    s = _stream_handle(x.device)
    with _on_device(x.device):
        skinny_gemm_bf16_split_k(x.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K, plan,
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(), s)
    return out


def gemm_split_k_noalloc(x: torch.Tensor, W: torch.Tensor, plan: Plan | None = None,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """y = x @ W.T with cross-block split-K on the library's static workspace
    (skinny_gemm_bf16_split_k_noalloc); with `out` given, nothing is allocated."""
    M, N, K, out = _split_args(x, W, out)
    s = _stream_handle(x.device)
    with _on_device(x.device):
        skinny_gemm_bf16_split_k_noalloc(x.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K, plan, s)
    return out


__all__ = [
    "SkinnyError", "Plan", "lib", "variants", "gemm", "gemm_pair", "gemm_pair_strided",
    "split_k_variants", "split_k_workspace", "gemm_split_k", "gemm_split_k_noalloc",
    "skinny_gemm_split_k_workspace_bytes", "skinny_gemm_bf16_split_k",
    "skinny_gemm_bf16_split_k_noalloc", "skinny_gemm_split_k_num_variants",
    "skinny_gemm_split_k_get_variant", "skinny_gemm_split_k_default_plan", "SKINNY_KIND_SPLIT_K",
    "skinny_gemm_bf16_pair_strided", "skinny_gemm_bf16_pair_strided_ex",
    "skinny_gemm_init", "skinny_gemm_bf16", "skinny_gemm_bf16_pair", "skinny_gemm_bf16_ex",
    "skinny_gemm_bf16_pair_ex", "skinny_gemm_bf16_f32out", "skinny_gemm_bf16_f32out_ex",
    "skinny_gemm_get_plan", "skinny_gemm_num_variants",
    "skinny_gemm_get_variant", "skinny_gemm_status_string", "skinny_gemm_version",
    "SKINNY_OK", "SKINNY_ERR_INVALID_ARG", "SKINNY_ERR_UNSUPPORTED", "SKINNY_ERR_NOT_INITIALIZED",
    "SKINNY_ERR_LAUNCH", "SKINNY_KIND_FIXED_K", "SKINNY_KIND_LOOP_K", "SKINNY_KIND_SCALAR",
    "SKINNY_KIND_MFMA",
]
