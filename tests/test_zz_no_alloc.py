"""skinny_gemm_bf16_split_k_noalloc, the split-K entry point that allocates
nothing (it uses the library's static per-GPU workspace), against
skinny_gemm_bf16_split_k with a caller-owned workspace, through the C ABI.

Both run the same kernel, so the outputs must agree bit for bit; each is also
held to the oracle's bar (oracle/accept.py). Two no-alloc calls run back to back,
the second on a smaller input, so the second finds the static workspace as the
first left it.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


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


def noalloc(skg, x, W, y, plan=None):
    M, K = x.shape
    N = W.shape[0]
    return skg.lib().skinny_gemm_bf16_split_k_noalloc(
        x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K,
        ctypes.byref(plan) if plan is not None else None, torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_workspace_entry(skg):
    cases = [(4096, 8192, 4), (1000, 4096, 2)]  # the second call is smaller
    data, refs = [], []
    for i, (N, K, M) in enumerate(cases):
        W = synth.weights(N, K, seed=21, shape_id=i)
        x = synth.activations(M, K, seed=21, shape_id=i)
        xd, Wd = to_dev(x), to_dev(W)
        ws = skg.split_k_workspace(M, N, K)
        refs.append(to_host(skg.gemm_split_k(xd, Wd, ws)))
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y.view(torch.int16).fill_(0x7FC0)  # NaN: any output left unwritten shows
        data.append((x, W, xd, Wd, y))
    torch.cuda.synchronize()
    for x, W, xd, Wd, y in data:
        assert noalloc(skg, xd, Wd, y) == skg.SKINNY_OK
    torch.cuda.synchronize()
    for (x, W, xd, Wd, y), ref, (N, K, M) in zip(data, refs, cases):
        got = to_host(y)
        assert np.array_equal(got, ref), f"({N},{K}) M={M}"
        yr, r64, mag = oracle.gemm(x, W)
        res = oracle.acceptance(got, yr, r64, mag)
        assert res["pass"], f"({N},{K}) M={M}: {res}"


def test_noalloc_with_explicit_plans_and_graph_replay(skg):
    """Every split count of one variant in a row, then the call replayed from a
    captured graph (the callers this entry point is for capture their calls)."""
    N, K, M = 2048, 4096, 3
    W = synth.weights(N, K, seed=22)
    x = synth.activations(M, K, seed=22)
    xd, Wd = to_dev(x), to_dev(W)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    for S, chunks in ((8, 1), (4, 2), (2, 4), (1, 8)):
        plan = skg.Plan(kind=skg.SKINNY_KIND_SPLIT_K, threads_per_block=256, lanes_per_row=64,
                        chunks=chunks, rows_per_wave=1, k_split=S, nontemporal=1, grid_blocks=0,
                        x_in_lds=0, prefetch=0)
        ws = skg.split_k_workspace(M, N, K, plan)
        ref = to_host(skg.gemm_split_k(xd, Wd, ws, plan=plan))
        y.view(torch.int16).fill_(0x7FC0)
        assert noalloc(skg, xd, Wd, y, plan) == skg.SKINNY_OK
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), ref), f"S={S}"
    eager = to_host(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            assert noalloc(skg, xd, Wd, y, plan) == skg.SKINNY_OK
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        y.view(torch.int16).fill_(0x7FC0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), eager), f"replay {rep}"


def test_noalloc_refuses_beyond_its_workspace(skg):
    """S*M*N above 2^20 floats, or more than 16384 row tiles: refused, nothing runs."""
    K = 4096
    plan = skg.skinny_gemm_split_k_default_plan(8, 32768, K)  # S = 4
    assert plan.k_split == 4
    W = torch.zeros((32769, K), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((8, K), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((8, 32769), dtype=torch.bfloat16, device="cuda")
    # 4 * 8 * 32768 = 2^20 floats: accepted; one row more is refused
    assert noalloc(skg, x, W[:32768], y[:, :32768].contiguous(), plan) == skg.SKINNY_OK
    assert noalloc(skg, x, W, y, plan) == skg.SKINNY_ERR_INVALID_ARG
    torch.cuda.synchronize()


_CAPTURE_FIRST = r"""
import sys
import torch
sys.path.insert(0, sys.argv[1])
import bf16_skinny_gemm_amd as skg
dev = torch.device("cuda:0")
torch.cuda.set_device(dev)
if sys.argv[2] == "init":
    skg.skinny_gemm_init(0)  # looks the workspace up; its counters are cleared by the first call
g0 = torch.Generator(device=dev).manual_seed(23)
N, K, M = 2048, 4096, 2
W = (torch.randn(N, K, device=dev, generator=g0) / 64).to(torch.bfloat16)
x = torch.randn(M, K, device=dev, generator=g0).to(torch.bfloat16)
y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
g = torch.cuda.CUDAGraph()
with torch.cuda.stream(s):
    with torch.cuda.graph(g, stream=s):
        st = skg.lib().skinny_gemm_bf16_split_k_noalloc(x.data_ptr(), W.data_ptr(), y.data_ptr(),
                                                        M, N, K, None, s.cuda_stream)
assert st == 0, st
torch.cuda.current_stream().wait_stream(s)
ref = skg.gemm_split_k(x, W, skg.split_k_workspace(M, N, K))
for r in range(3):
    y.view(torch.int16).fill_(0x7FC0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), r
print("ok")
"""


@pytest.mark.parametrize("setup", ["init", "lazy"])
def test_noalloc_first_call_inside_graph_capture(skg, setup):
    """A fresh process whose first no-alloc call is made under graph capture, after
    skinny_gemm_init (which looked the workspace up) or without it (the call looks it
    up): the counter-clearing kernel of the first call lands in the graph, and every
    replay gives the workspace entry point's bits."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print(f"fresh process ({setup}): first no-alloc call under capture, (2048,4096) M=2", flush=True)
    res = subprocess.run([sys.executable, "-c", _CAPTURE_FIRST, root, setup], capture_output=True,
                         text=True, timeout=240)
    assert res.returncode == 0 and "ok" in res.stdout, res.stdout + res.stderr[-3000:]
