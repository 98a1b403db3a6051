"""Build libfp8q.so (gfx950) in-tree with hipcc.

Usage: python fine_grained_block_fp8q_amd/build.py   (or load this file and
call build(); importing it through the package would first load the library
it builds).  The library lands next to this file; the Python binding loads it
from there.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8q.so")
# The same sources with FP8Q_DEBUG_CHECKS: grouped calls synchronize after the
# launch and report invalid device offsets as FP8Q_ERR_OFFSETS.
LIB_DEBUG = os.path.join(PKG, "libfp8q_debug.so")
# Measurement support for bench.py --copy-probe (streaming-bandwidth ceiling
# and counter calibration); not part of the method's C ABI.
LIB_PROBE = os.path.join(PKG, "libfp8q_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # no packed-FP32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source extra flags.  The quantizer's codes are a bit-exact contract:
# no FP contraction and no fast math there.
SOURCES = {
    "quant_kernels.hip": ["-ffp-contract=off"],
    # keep MFMA results in arch VGPRs: the promotion FMAs read them directly
    # instead of copying each element out of an AGPR first; let the main
    # loop's step sequence unroll fully also with the activation cast in it
    # (left rolled, its register arrays would go to scratch memory)
    "gemm_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                         "-mllvm", "-pragma-unroll-threshold=60000"],
    "fp8q_api.hip": [],
}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def _build_one(lib, tag, defines, verbose):
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD_DIR, src.replace(".hip", f"{tag}.o"))
        cmd = [HIPCC, *COMMON, *defines, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = lib + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every HIP source for gfx950 and link libfp8q.so and its
    FP8Q_DEBUG_CHECKS variant libfp8q_debug.so (always rebuilds)."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(3) as ex:
        jobs = [ex.submit(_build_one, LIB, "", [], verbose),
                ex.submit(_build_one, LIB_DEBUG, "_debug", ["-DFP8Q_DEBUG_CHECKS"], verbose),
                ex.submit(_build_probe, verbose)]
        for j in jobs:
            j.result()
    return LIB


def _build_probe(verbose):
    tmp = LIB_PROBE + ".tmp"
    out = _run([HIPCC, *COMMON, "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-shared",
                os.path.join(CSRC, "stream_probe.hip"), os.path.join(CSRC, "mix_probe.hip"),
                os.path.join(CSRC, "ring_probe.hip"),
                "-o", tmp])
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PROBE)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
