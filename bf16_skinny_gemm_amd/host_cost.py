"""Eager host cost of one skinny GEMM call, per layer of the stack.

    python -m bf16_skinny_gemm_amd.host_cost [--shape N,K] [--M 1] [--calls 1000]

vLLM PR #65306 (SM90 skinny GEMM plans), section Details, puts the eager
custom-op overhead of its skinny GEMM at 4-7 µs per call; under graph replay it
is zero. This measures the same thing here: the wall time a Python caller spends
per call to enqueue one launch, with the GPU kept busy by a long spin kernel
issued first, so that no call waits for the device and the figure is host time
only. Layers timed, each over `--calls` back-to-back calls, median of 7 rounds:

  ctypes_floor   a C entry point that does nothing (skinny_gemm_version): the
                 ctypes call itself
  c_abi_reject   skinny_gemm_bf16 refused by its argument check (M = 9): ctypes
                 plus validation
  c_abi          skinny_gemm_bf16 on raw device pointers and a stream handle
  skg_gemm_out   bf16_skinny_gemm_amd.gemm(x, W, out=y)
  skg_gemm       bf16_skinny_gemm_amd.gemm(x, W) (allocates y)
  torch_op       torch.ops.skinny.linear(x, W)
  f_linear       torch.nn.functional.linear(x, W) (the vendor path, for scale)

The first call of a shape resolves its launch (plan lookup, occupancy query) and
caches it; `first_call_us` is that call alone.
"""
from __future__ import annotations

import argparse
import json
import statistics
import sys
import time


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shape", default="4096,4096")
    ap.add_argument("--M", type=int, default=1)
    ap.add_argument("--calls", type=int, default=1000)
    ap.add_argument("--rounds", type=int, default=7)
    args = ap.parse_args(argv)

    import torch

    import bf16_skinny_gemm_amd as skg
    from bf16_skinny_gemm_amd import torch_op  # noqa: F401  (registers torch.ops.skinny.linear)

    if not torch.cuda.is_available():
        print("host_cost needs a GPU", file=sys.stderr)
        return 1
    N, K = (int(v) for v in args.shape.split(","))
    M = args.M
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    skg.skinny_gemm_init(0)
    x = torch.randn((M, K), device=dev).to(torch.bfloat16)
    W = (torch.randn((N, K), device=dev) / K ** 0.5).to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    L = skg.lib()
    stream = torch.cuda.current_stream().cuda_stream
    xp, wp, yp = x.data_ptr(), W.data_ptr(), y.data_ptr()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    skg.skinny_gemm_bf16(xp, wp, yp, M, N, K, stream)
    first = (time.perf_counter() - t0) * 1e6
    torch.cuda.synchronize()

    layers = {
        "ctypes_floor": lambda: L.skinny_gemm_version(),
        "c_abi_reject": lambda: L.skinny_gemm_bf16(xp, wp, yp, 9, N, K, stream),
        "c_abi": lambda: L.skinny_gemm_bf16(xp, wp, yp, M, N, K, stream),
        "skg_gemm_out": lambda: skg.gemm(x, W, out=y),
        "skg_gemm": lambda: skg.gemm(x, W),
        "torch_op": lambda: torch.ops.skinny.linear(x, W),
        "f_linear": lambda: torch.nn.functional.linear(x, W),
    }
    out = {"shape": [N, K], "M": M, "calls_per_round": args.calls, "rounds": args.rounds,
           "first_call_us": round(first, 2), "us_per_call": {}}
    for name, fn in layers.items():
        for _ in range(20):  # warm-up (and the torch op's first dispatch)
            fn()
        torch.cuda.synchronize()
        per = []
        for _ in range(args.rounds):
            torch.cuda._sleep(200_000_000)  # keep the GPU busy: no call waits for it
            t0 = time.perf_counter()
            for _ in range(args.calls):
                fn()
            per.append((time.perf_counter() - t0) * 1e6 / args.calls)
            torch.cuda.synchronize()
        out["us_per_call"][name] = round(statistics.median(per), 3)
        print(f"{name:14s} {out['us_per_call'][name]:8.3f} us per call", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
