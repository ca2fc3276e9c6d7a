"""Seeded synthetic inputs for the BF16 skinny GEMM, shared by the oracle side and
the HIP side.

This module only *draws* inputs. It holds none of the GEMM's arithmetic: values
are sampled in float32 with numpy's PCG64 and turned into bfloat16 by torch's
own float32 -> bfloat16 conversion (round to nearest even), then handed out as
raw uint16 bit patterns. Nothing here multiplies, accumulates or rounds an
output.

Workload recipe (the decode projections of vLLM PR #62949, SM121 skinny GEMM
plans, section Validation): activations x ~ N(0, 1), weights W ~ N(0, 1/K), i.e.
standard deviation 1/sqrt(K), row-major, seed 0, one independent stream per
tensor derived as ``default_rng([seed, shape_id, tensor_id])``.

vLLM PR #65306 (SM90 skinny GEMM plans), section Validation, also checks
outlier and scaled/sparse inputs without defining them; the reading used here
is: outlier = 1% of x's K channels multiplied by 64, scaled = x times 2**s,
sparse = 90% of x's entries set to zero.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "normal_bf16",
    "activations",
    "weights",
    "outlier_activations",
    "scaled_activations",
    "sparse_activations",
    "small_int_bf16",
    "device_weights",
    "BF16_ONE",
]

BF16_ONE = np.uint16(0x3F80)  # bit pattern of 1.0 in bfloat16


def rng(seed: int, *stream_ids: int) -> np.random.Generator:
    """Independent PCG64 stream for (seed, *stream_ids)."""
    return np.random.default_rng([int(seed), *[int(s) for s in stream_ids]])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), via torch's conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact widening)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, std: float, g: np.random.Generator) -> np.ndarray:
    """N(0, std^2) samples drawn in float32, scaled in float32, stored as bf16 bits."""
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def activations(M: int, K: int, seed: int = 0, shape_id: int = 0, tensor_id: int = 0) -> np.ndarray:
    """x[M, K] ~ N(0, 1) as bf16 bits."""
    return normal_bf16((M, K), 1.0, rng(seed, shape_id, tensor_id))


def weights(N: int, K: int, seed: int = 0, shape_id: int = 0, tensor_id: int = 1) -> np.ndarray:
    """W[N, K] ~ N(0, 1/K) as bf16 bits (row-major, nn.Linear layout)."""
    return normal_bf16((N, K), 1.0 / np.sqrt(K), rng(seed, shape_id, tensor_id))


def outlier_activations(M: int, K: int, seed: int = 0, shape_id: int = 0, tensor_id: int = 0,
                        frac: float = 0.01, factor: float = 64.0) -> np.ndarray:
    """x ~ N(0,1) with a seeded 1% of the K channels multiplied by 64."""
    g = rng(seed, shape_id, tensor_id, 101)
    a = g.standard_normal(size=(M, K), dtype=np.float32)
    n_out = max(1, int(round(frac * K)))
    cols = g.choice(K, size=n_out, replace=False)
    a[:, cols] *= np.float32(factor)
    return f32_to_bf16_bits(a)


def scaled_activations(M: int, K: int, log2_scale: int, seed: int = 0, shape_id: int = 0,
                       tensor_id: int = 0) -> np.ndarray:
    """x ~ N(0,1) times 2**log2_scale (exact power-of-two scaling in float32)."""
    g = rng(seed, shape_id, tensor_id, 102)
    a = g.standard_normal(size=(M, K), dtype=np.float32)
    a *= np.float32(2.0 ** log2_scale)
    return f32_to_bf16_bits(a)


def sparse_activations(M: int, K: int, seed: int = 0, shape_id: int = 0, tensor_id: int = 0,
                       zero_frac: float = 0.9) -> np.ndarray:
    """x ~ N(0,1) with a seeded 90% of the entries set to zero."""
    g = rng(seed, shape_id, tensor_id, 103)
    a = g.standard_normal(size=(M, K), dtype=np.float32)
    a[g.random(size=(M, K)) < zero_frac] = 0.0
    return f32_to_bf16_bits(a)


def small_int_bf16(shape, lo: int, hi: int, g: np.random.Generator) -> np.ndarray:
    """Uniform integers in [lo, hi] as bf16 bits (exact for |v| <= 256)."""
    a = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(a)


def device_weights(N: int, K: int, seed: int, tensor_id: int, device):
    """W[N, K] ~ N(0, 1/K) drawn on the GPU, as a bfloat16 torch tensor.

    For the decode-step chain, whose 186 distinct weights (7.5 GB) would take
    minutes through numpy: torch's Philox generator on `device`, seeded with
    ``seed * 1_000_003 + tensor_id``, draws float32 standard normals, they are
    scaled by 1/sqrt(K) in float32 and rounded to bfloat16 by torch's
    nearest-even conversion. The same bits serve both sides: the oracle reads a
    host copy of the tensor, the kernels the tensor itself.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(tensor_id))
    a = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    a.mul_(float(np.float32(1.0 / np.sqrt(K))))
    return a.to(torch.bfloat16)
