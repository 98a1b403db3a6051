"""Device-side validation of the grouped calls' offsets (0 = off[0] <= ... <=
off[G] <= M_total), through the C ABI of both builds:
- libfp8q.so: a launch with invalid offsets writes nothing (the output keeps
  its contents) and the call returns FP8Q_OK (the check runs on the device);
- libfp8q_debug.so (FP8Q_DEBUG_CHECKS): the call synchronizes and returns
  FP8Q_ERR_OFFSETS, and valid calls still give the release library's output
  bit for bit.
Every buffer holds more rows than any of the offsets below reaches, so no
access could leave the allocations even if a launch ignored its check.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_util import DEV, fq

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DEBUG = os.path.join(ROOT, "fine_grained_block_fp8q_amd", "libfp8q_debug.so")
OK, E_OFFSETS = 0, 8
G, N, K, ROWS = 3, 256, 384, 512        # physical rows of every row-indexed buffer


def _debug_lib():
    L = ctypes.CDLL(LIB_DEBUG)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    for name in ("fp8q_grouped_gemm", "fp8q_grouped_gemm_precise"):
        getattr(L, name).argtypes = [p, p, i64, p, i32, p, p, i64, i64, p, i32, p]
        getattr(L, name).restype = ctypes.c_int
    L.fp8q_grouped_gemm_fused.argtypes = [p, i64, p, i32, p, p, i64, i64, p, i32, i32, p]
    L.fp8q_grouped_gemm_fused.restype = ctypes.c_int
    L.fp8q_debug_checks.restype = ctypes.c_int
    assert L.fp8q_debug_checks() == 1
    return L


@pytest.fixture(scope="module")
def bufs():
    f = fq()
    g = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn((ROWS, K), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((G * N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    aq, as_ = f.quantize_act(x)            # [ROWS][K], [K/128][ROWS]
    wq, ws = f.quantize_weight(w)
    return x, aq, as_, wq.view(G, N, K), ws.view(G, N // 128, K // 128)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _call(L, name, bufs, off, M_total, c):
    x, aq, as_, wq, ws = bufs
    d_off = torch.tensor(off, dtype=torch.int32, device=DEV)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if name == "fp8q_grouped_gemm_fused":
        st = L.fp8q_grouped_gemm_fused(_ptr(x), M_total, _ptr(d_off), G, _ptr(wq), _ptr(ws), N, K,
                                       _ptr(c), 0, 0, s)
    else:
        # a_s is [K/128][ROWS]: a leading dimension of M_total is passed only
        # for M_total == ROWS; the invalid cases below never run a tile
        st = getattr(L, name)(_ptr(aq), _ptr(as_), M_total, _ptr(d_off), G, _ptr(wq), _ptr(ws),
                              N, K, _ptr(c), 0, s)
    torch.cuda.synchronize()
    return st


BAD = {
    "decreasing": [0, 80, 40, 100],
    "past_M_total": [0, 60, 90, 130],     # M_total = 100 below
    "nonzero_start": [10, 50, 70, 100],
}
NAMES = ["fp8q_grouped_gemm", "fp8q_grouped_gemm_precise", "fp8q_grouped_gemm_fused"]


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("case", list(BAD))
def test_release_build_writes_nothing_for_invalid_offsets(bufs, name, case):
    c = torch.full((ROWS, N), float("nan"), dtype=torch.float32, device=DEV)
    st = _call(fq().lib, name, bufs, BAD[case], 100, c)
    assert st == OK
    assert torch.isnan(c).all(), "a launch with invalid offsets must leave the output untouched"


@pytest.mark.parametrize("name", NAMES)
def test_debug_build_reports_invalid_offsets(bufs, name):
    L = _debug_lib()
    for case, off in BAD.items():
        c = torch.full((ROWS, N), float("nan"), dtype=torch.float32, device=DEV)
        assert _call(L, name, bufs, off, 100, c) == E_OFFSETS, case
        assert torch.isnan(c).all(), case
    # valid offsets (an empty expert included): OK, and the release build's
    # output bit for bit; the error flag was cleared by the reporting call
    off = [0, 200, 200, ROWS]
    c_dbg = torch.full((ROWS, N), float("nan"), dtype=torch.float32, device=DEV)
    c_rel = torch.full((ROWS, N), float("nan"), dtype=torch.float32, device=DEV)
    assert _call(L, name, bufs, off, ROWS, c_dbg) == OK
    assert _call(fq().lib, name, bufs, off, ROWS, c_rel) == OK
    assert not torch.isnan(c_rel).any()
    assert torch.equal(c_dbg.view(torch.int32), c_rel.view(torch.int32))
