"""PyTorch operator and module hook for the skinny GEMM.

The routing follows the plan-table hook of vLLM PR #62949 (SM121 skinny GEMM
plans, sections Claims and Details) and vLLM PR #65306 (SM90 skinny GEMM plans,
section Details): a linear layer's apply path takes the skinny GEMM when the GPU
architecture, the dtype and the token count qualify, and keeps the standard
linear path otherwise. Here:

* ``torch.ops.skinny.linear(x, weight)`` is a custom operator (graph-capturable,
  with a fake implementation for tracing) that always runs the HIP kernel and
  raises if the call does not qualify. Its GPU and CPU implementations are
  registered in C++ (``libskinny_torch_op.so``, built from csrc/torch_op.cpp), so
  an eager call goes from the dispatcher to the C ABI with no Python frame; when
  that library has not been built, the same operator is registered from Python
  below (it calls the same C entry point through ctypes, at a few µs more per
  eager call);
* :func:`skinny_linear` routes: qualifying calls go to the op, others to
  ``torch.nn.functional.linear`` only when ``fallback=True`` (the default for the
  module hook), else they raise;
* :func:`install` swaps the forward of ``nn.Linear`` modules for the routed one.

A call qualifies when x and weight are bfloat16 CUDA tensors on a gfx950 device,
weight is [N, K] contiguous, x is [..., K] with 1 <= prod(leading dims) <= 8
(the token count M: the cited pages route 1..4; 5..8 is routed here too, since on
MI355X the kernels measured faster than F.linear there on the decode shapes), and
there is no bias. The kernel itself never falls back: a missing library or a
refused launch raises.
"""
from __future__ import annotations

import functools
import os

import torch

from . import _on_device, _stream_handle, lib, skinny_gemm_bf16
from .build import TORCH_OP_PATH

_ARCH_OK: dict[int, bool] = {}


def _device_is_gfx950(device: torch.device) -> bool:
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _ARCH_OK:
        props = torch.cuda.get_device_properties(idx)
        _ARCH_OK[idx] = str(getattr(props, "gcnArchName", "")).startswith("gfx950")
    return _ARCH_OK[idx]


def qualifies(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None) -> bool:
    """True when (x, weight, bias) can run on the skinny GEMM."""
    if bias is not None:
        return False
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        return False
    if x.device.type != "cuda" or weight.device != x.device:
        return False
    if weight.dim() != 2 or x.dim() < 1 or x.shape[-1] != weight.shape[1]:
        return False
    if not weight.is_contiguous():
        # a strided weight would have to be copied whole on every call (634 MB for
        # the LM head): leave it to the standard path
        return False
    m = 1
    for d in x.shape[:-1]:
        m *= d
    if not (1 <= m <= 8):
        return False
    return _device_is_gfx950(x.device)


def _linear_gpu(x: torch.Tensor, weight: torch.Tensor) -> torch.Tensor:
    """y = x @ weight.T on the HIP skinny GEMM; x [..., K] with M = prod(...) <= 8."""
    if not qualifies(x, weight):
        raise ValueError("skinny::linear: inputs do not qualify (bf16 on gfx950, no bias, "
                         f"M in 1..8): x {tuple(x.shape)} {x.dtype}, weight "
                         f"{tuple(weight.shape)} {weight.dtype}")
    K = x.shape[-1]
    N = weight.shape[0]
    x2 = x.reshape(-1, K)
    if not x2.is_contiguous():
        x2 = x2.contiguous()
    y = torch.empty((*x.shape[:-1], N), dtype=torch.bfloat16, device=x.device)
    # qualifies() has checked dtypes, devices and shapes: call the C entry point
    # directly (it raises if the library is missing or refuses the call)
    with _on_device(x.device):
        skinny_gemm_bf16(x2.data_ptr(), weight.data_ptr(), y.data_ptr(), x2.shape[0], N, K,
                         _stream_handle(x.device))
    return y


def _linear_other(x: torch.Tensor, weight: torch.Tensor) -> torch.Tensor:
    raise ValueError("skinny::linear: runs on gfx950 GPU tensors only, got "
                     f"x on {x.device}, weight on {weight.device}")


def _linear_fake(x: torch.Tensor, weight: torch.Tensor) -> torch.Tensor:
    return x.new_empty((*x.shape[:-1], weight.shape[0]))


if os.path.exists(TORCH_OP_PATH):
    # the C++ registration: schema and the CUDA / CPU kernels; the GEMM library it
    # links is the one the ctypes binding loads (same file, one copy in the process)
    lib()
    torch.ops.load_library(TORCH_OP_PATH)
    _LIB = torch.library.Library("skinny", "FRAGMENT")
    CPP_OP = True
else:
    # The Python registration goes through torch.library.Library rather than the
    # torch.library.custom_op decorator: the decorator's Python wrapping costs about
    # 10 us per eager call on its own, the plain registration about 3 us.
    _LIB = torch.library.Library("skinny", "DEF")
    _LIB.define("linear(Tensor x, Tensor weight) -> Tensor")
    _LIB.impl("linear", _linear_gpu, "CUDA")
    _LIB.impl("linear", _linear_other, "CPU")
    CPP_OP = False
torch.library.register_fake("skinny::linear", _linear_fake, lib=_LIB)
linear = torch.ops.skinny.linear


def skinny_linear(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
                  fallback: bool = True) -> torch.Tensor:
    """F.linear semantics, routed: the skinny GEMM when the call qualifies,
    otherwise torch.nn.functional.linear if ``fallback`` (else ValueError)."""
    if qualifies(x, weight, bias):
        return torch.ops.skinny.linear(x, weight)
    if not fallback:
        raise ValueError("skinny_linear: call does not qualify for the skinny GEMM")
    return torch.nn.functional.linear(x, weight, bias)


def install(module: torch.nn.Module, fallback: bool = True) -> int:
    """Route the forward of every nn.Linear inside ``module`` through
    :func:`skinny_linear`. Returns the number of layers hooked."""
    count = 0
    for sub in module.modules():
        if isinstance(sub, torch.nn.Linear) and not getattr(sub, "_skinny_hooked", False):
            def fwd(self, inp, _fallback=fallback):
                return skinny_linear(inp, self.weight, self.bias, fallback=_fallback)
            sub.forward = functools.partial(fwd, sub)
            sub._skinny_hooked = True
            count += 1
    return count


__all__ = ["linear", "skinny_linear", "install", "qualifies", "CPP_OP"]
