"""The C ABI from C: tests/c/abi_check.c is compiled as C99 with gcc against
include/fp8q.h, linked to libfp8q.so and run (no GPU needed: it checks the
ABI version, a status string, empty no-ops and the host-side validation
codes of every GEMM entry point)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "fine_grained_block_fp8q_amd")
ROCM_INCLUDE = "/opt/rocm/include"


def test_c_program_against_the_header_and_library(tmp_path):
    if shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("gcc or the ROCm headers are not installed")
    if not os.path.exists(os.path.join(LIBDIR, "libfp8q.so")):
        pytest.fail("libfp8q.so is not built (python fine_grained_block_fp8q_amd/build.py)")
    exe = str(tmp_path / "abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", exe,
           "-L", LIBDIR, "-lfp8q", "-Wl,-rpath," + LIBDIR]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60,
                         env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c abi ok" in run.stdout
