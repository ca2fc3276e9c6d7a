"""Build libskinny_gemm_bf16.so in-tree with hipcc for gfx950.

    python -m bf16_skinny_gemm_amd.build

The library is built next to this file so that it travels with the source
tree; it is never installed into site-packages. Its translation units (the host
side and the variant tables, which hold the kernel instances) are compiled in
parallel into objects under _build/ and linked once. The read-stream probe used
by the benchmark (include/skinny_stream_probe.h) is built beside it as
libskinny_stream_probe.so, and the torch operator (csrc/torch_op.cpp) as
libskinny_torch_op.so, with the host compiler against torch's headers.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libskinny_gemm_bf16.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"
SOURCES = ("skinny_gemm.hip", "variants_fixed_small.hip", "variants_fixed_k4096.hip",
           "variants_fixed_k8192.hip", "variants_other.hip", "split_k.hip")
PROBE_LIB_PATH = os.path.join(HERE, "libskinny_stream_probe.so")
# torch.ops.skinny.linear with its GPU kernel registered in C++ (a host-only
# translation unit built with the host compiler against torch's headers; it
# links the GEMM library above)
TORCH_OP_PATH = os.path.join(HERE, "libskinny_torch_op.so")
TORCH_OP_SOURCE = "torch_op.cpp"
PROBE_SOURCES = ("stream_probe.hip",)

# hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
_NOISE = ("packed-fp32-ops", "not a recognized feature for this target")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_command(src: str, obj: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
        # packed-FP32 instructions are left to no one: the compiler must not form them
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-I", INCLUDE, "-I", CSRC,
        "-o", obj, os.path.join(CSRC, src),
    ]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs]


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in _NOISE))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    return err


def build_library(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile the HIP library and the read-stream probe (always recompiles) and
    return the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tag = f".{os.getpid()}"
    sources = SOURCES + PROBE_SOURCES
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + tag + ".o") for s in sources]
    workers = jobs or max(1, min(len(sources), os.cpu_count() or 1))
    outs = ((LIB_PATH, objs[:len(SOURCES)]), (PROBE_LIB_PATH, objs[len(SOURCES):]))
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            errs = list(pool.map(_run, [compile_command(s, o) for s, o in zip(sources, objs)]))
        for path, part in outs:
            errs.append(_run(link_command(part, path + f".tmp{os.getpid()}")))
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    if verbose:
        for e in errs:
            if e.strip():
                print(e, file=sys.stderr)
    for path, _ in outs:
        os.replace(path + f".tmp{os.getpid()}", path)
    return LIB_PATH


def torch_op_commands(obj: str, out: str) -> list[list[str]]:
    """g++ compile and link lines of the torch operator library."""
    import torch
    import torch.utils.cpp_extension as ce

    abi = "1" if torch.compiled_with_cxx11_abi() else "0"
    incs = [f"-I{d}" for d in ce.include_paths(device_type="cuda")] + ["-I", INCLUDE]
    libs = ce.library_paths(device_type="cuda")
    compile_cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", f"-D_GLIBCXX_USE_CXX11_ABI={abi}",
                   "-DUSE_ROCM=1", "-D__HIP_PLATFORM_AMD__=1", *incs, "-c",
                   os.path.join(CSRC, TORCH_OP_SOURCE), "-o", obj]
    link_cmd = ["g++", "-shared", "-o", out, obj, f"-L{HERE}", "-lskinny_gemm_bf16",
                *[f"-L{d}" for d in libs], "-lc10", "-lc10_hip", "-ltorch", "-ltorch_cpu",
                "-ltorch_hip", "-lamdhip64", "-Wl,-rpath,$ORIGIN", *[f"-Wl,-rpath,{d}" for d in libs[:1]]]
    return [compile_cmd, link_cmd]


def build_torch_op(verbose: bool = False) -> str:
    """Compile libskinny_torch_op.so (always recompiles); needs the GEMM library."""
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the GEMM library first")
    os.makedirs(BUILD_DIR, exist_ok=True)
    tag = f".{os.getpid()}"
    obj = os.path.join(BUILD_DIR, "torch_op" + tag + ".o")
    tmp = TORCH_OP_PATH + f".tmp{os.getpid()}"
    try:
        for cmd in torch_op_commands(obj, tmp):
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"building the torch op failed ({res.returncode}):\n{' '.join(cmd)}\n"
                                   f"{res.stderr[-6000:]}")
            if verbose and res.stderr.strip():
                print(res.stderr, file=sys.stderr)
        os.replace(tmp, TORCH_OP_PATH)
    finally:
        for f in (obj, tmp):
            if os.path.exists(f):
                os.remove(f)
    return TORCH_OP_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_torch_op(verbose=True))
