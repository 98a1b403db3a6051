"""Build and load the oracle's one C part (truncation_bound.c -> libtbound.so).

TEST INFRASTRUCTURE ONLY (see the package docstring).  __graft_entry__.build()
compiles it with the HIP library; a test that finds it missing builds it here
first (gcc).  No floating-point contraction: the C loop reproduces the NumPy
truncation bound bit for bit.
"""

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "truncation_bound.c")
LIB = os.path.join(HERE, "libtbound.so")


def build():
    """Compile truncation_bound.c into libtbound.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O3", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Werror", SRC, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stdout}")
    os.replace(tmp, LIB)


def load():
    """The loaded library, built first if it is not there."""
    if not os.path.exists(LIB):
        build()
    return ctypes.CDLL(LIB)
