"""Build libskinny_gemm_bf16.so in-tree with hipcc for gfx950.

    python -m bf16_skinny_gemm_amd.build

The library is built next to this file so that it travels with the source
tree; it is never installed into site-packages.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libskinny_gemm_bf16.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_command(out: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed-FP32 instructions are left to no one: the compiler must not form them
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-I", INCLUDE, "-I", CSRC,
        "-o", out, os.path.join(CSRC, "skinny_gemm.hip"),
    ]


def build_library(verbose: bool = False) -> str:
    """Compile the HIP library (always recompiles) and return its path."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
    noise = ("packed-fp32-ops", "not a recognized feature for this target")
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
