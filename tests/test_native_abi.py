"""The C ABI used from C++ with no Python in between: tests/native/abi_native.cpp
calls include/skinny_gemm.h on hipMalloc memory and checks every output against
the CPU oracle linked into it (G1, S1 and the row cosine), the argument checks'
refusals, the bit-exact replay of a captured graph, and split-K on a hipMalloc
workspace and on the library's static one."""
from __future__ import annotations

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "native", "abi_native")


def _exe() -> str:
    if not os.path.exists(EXE):
        import importlib.util

        spec = importlib.util.spec_from_file_location(
            "build_native", os.path.join(HERE, "native", "build_native.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build_native()
    return EXE


def test_native_program_links_and_refuses_without_gpu():
    """Without a visible GPU the program links, loads the library and exits 2."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the full program runs in the gpu test")
    res = subprocess.run([_exe()], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "no GPU" in res.stderr, (res.returncode, res.stderr)


@pytest.mark.gpu
def test_native_program_passes():
    print("native ABI program: shapes (4096,1024) (1000,1024) (2048,4096) (300,1536) (77,1000), "
          "M 1..8, pair, strided pair, refusals, graph replay, split-K with a workspace and without",
          flush=True)
    res = subprocess.run([_exe()], capture_output=True, text=True, timeout=180)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert "0 failures" in res.stdout
