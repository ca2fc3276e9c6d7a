"""Build tests/native/abi_native: a C++ consumer of include/skinny_gemm.h.

The program is compiled with hipcc (host code only), the CPU oracle's C source is
compiled into it with gcc under the oracle's own flags, and it links the in-tree
libskinny_gemm_bf16.so by an rpath relative to the executable. Run `python tests/native/build_native.py` after
the library is built; __graft_entry__.build() calls build_native() itself.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "abi_native")
LIB_DIR = os.path.join(ROOT, "bf16_skinny_gemm_amd")


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_native() -> str:
    tag = f".{os.getpid()}"
    oracle_obj = os.path.join(HERE, "skinny_oracle" + tag + ".o")
    main_obj = os.path.join(HERE, "abi_native" + tag + ".o")
    out = EXE + tag
    try:
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-c",
                        os.path.join(ROOT, "oracle", "skinny_oracle.c"), "-o", oracle_obj],
                       check=True)
        # compile and link in two steps: hipcc's source-language flag would also
        # apply to an object file named on the same line
        for cmd in ([_hipcc(), "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-c",
                     os.path.join(HERE, "abi_native.cpp"), "-o", main_obj],
                    [_hipcc(), main_obj, oracle_obj, "-L", LIB_DIR, "-lskinny_gemm_bf16",
                     "-Wl,-rpath,$ORIGIN/../../bf16_skinny_gemm_amd", "-lpthread", "-o", out]):
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"building abi_native failed:\n{' '.join(cmd)}\n{res.stderr[-4000:]}")
        os.replace(out, EXE)
    finally:
        for p in (oracle_obj, main_obj, out):
            if os.path.exists(p):
                os.remove(p)
    return EXE


if __name__ == "__main__":
    print(build_native())
    sys.exit(0)
