"""CPU sanitizer builds: the oracle and the C ABI's host-side argument checks
compiled with -fsanitize=address,undefined (gcc / g++, host code only) and run
over random and extreme inputs (tests/sanitize/). Any memory error or undefined
behaviour aborts the fuzzing program (-fno-sanitize-recover=all)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=300)
    return res.returncode, res.stdout + res.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    rc, out = _run(["gcc", "-std=c11", "-ffp-contract=off", "-pthread", *SAN,
                    os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"),
                    os.path.join(ROOT, "oracle", "skinny_oracle.c"), "-lm", "-o", exe], ROOT)
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "validate_fuzz")
    # the ABI header includes hip_runtime_api.h (for hipStream_t); g++ reads it as
    # the AMD platform's C API
    rc, out = _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "bf16_skinny_gemm_amd", "csrc"), "-I", "/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "sanitize", "validate_fuzz.cpp"),
                    "-o", exe], ROOT)
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "0 failures" in out
