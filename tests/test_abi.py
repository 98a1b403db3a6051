"""C-ABI checks that need no GPU: the library loads, exports every function
include/fp8q.h declares, and rejects invalid arguments on the host with the
documented status codes before touching any device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")
LIB = os.path.join(ROOT, "fine_grained_block_fp8q_amd", "libfp8q.so")
LIB_DEBUG = os.path.join(ROOT, "fine_grained_block_fp8q_amd", "libfp8q_debug.so")

OK, E_NULL, E_SHAPE, E_ALIGN, E_ENUM, E_DEVICE, E_LAUNCH, E_UNSUP, E_OFFSETS = range(9)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8q_[a-z0-9_]+)\s*\(", text)))


def _load(path):
    if not os.path.exists(path):
        pytest.fail(f"{os.path.basename(path)} is not built (python fine_grained_block_fp8q_amd/build.py)")
    L = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.fp8q_quantize_act.argtypes = [p, i64, i64, p, p, i32, p]
    L.fp8q_quantize_weight.argtypes = [p, i64, i64, p, p, i32, p]
    L.fp8q_gemm.argtypes = [p, p, p, p, i64, i64, i64, p, i32, p]
    L.fp8q_gemm_precise.argtypes = [p, p, p, p, i64, i64, i64, p, i32, p]
    L.fp8q_gemm_mfma_scaled.argtypes = [p, p, p, p, i64, i64, i64, p, i32, p]
    L.fp8q_grouped_gemm.argtypes = [p, p, i64, p, i32, p, p, i64, i64, p, i32, p]
    L.fp8q_grouped_gemm_precise.argtypes = [p, p, i64, p, i32, p, p, i64, i64, p, i32, p]
    L.fp8q_gemm_rowscaled_precise.argtypes = [p, p, p, p, i64, i64, i64, p, i32, p]
    L.fp8q_gemm_bf16.argtypes = [p, p, i64, i64, i64, p, i32, p]
    L.fp8q_quantize_act_t.argtypes = [p, i64, i64, p, p, i32, p]
    L.fp8q_quantize_weight_t.argtypes = [p, i64, i64, p, p, i32, p]
    L.fp8q_gemm_rowscaled.argtypes = [p, p, p, p, i64, i64, i64, p, i32, p]
    L.fp8q_gemm_fused.argtypes = [p, p, p, i64, i64, i64, p, i32, i32, p]
    L.fp8q_grouped_gemm_fused.argtypes = [p, i64, p, i32, p, p, i64, i64, p, i32, i32, p]
    L.fp8q_status_string.restype = ctypes.c_char_p
    L.fp8q_status_string.argtypes = [ctypes.c_int]
    return L


@pytest.fixture(scope="module", params=["release", "debug_checks"])
def lib(request):
    """Both builds: the library and its FP8Q_DEBUG_CHECKS variant validate
    arguments on the host identically."""
    return _load(LIB if request.param == "release" else LIB_DEBUG)


def _no_device():
    """True when no GPU is visible (the fake pointers below must never reach a
    kernel).  device_count() does not initialise the GPU."""
    import torch
    return torch.cuda.device_count() == 0


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) >= {"fp8q_quantize_act", "fp8q_quantize_weight", "fp8q_gemm",
                          "fp8q_gemm_precise", "fp8q_gemm_mfma_scaled", "fp8q_grouped_gemm",
                          "fp8q_grouped_gemm_precise",
                          "fp8q_gemm_bf16", "fp8q_quantize_act_t", "fp8q_quantize_weight_t",
                          "fp8q_gemm_rowscaled", "fp8q_gemm_rowscaled_precise", "fp8q_gemm_fused",
                          "fp8q_grouped_gemm_fused", "fp8q_status_string", "fp8q_abi_version",
                          "fp8q_debug_checks"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.fp8q_abi_version() == 3
    assert lib.fp8q_debug_checks() in (0, 1)
    for s in range(9):
        txt = lib.fp8q_status_string(s).decode()
        assert txt.startswith("FP8Q_")
    assert "UNKNOWN" in lib.fp8q_status_string(99).decode()


A = 0x10000  # fake, 64 KiB-aligned "device" addresses: never dereferenced on these paths


def test_quantize_act_validation(lib):
    f = lib.fp8q_quantize_act
    assert f(None, 4, 128, A, A, 0, None) == E_NULL
    assert f(A, 4, 128, None, A, 0, None) == E_NULL
    assert f(A, 4, 128, A, None, 0, None) == E_NULL
    assert f(None, 0, 128, None, None, 0, None) == OK  # empty is a no-op
    assert f(A, -1, 128, A, A, 0, None) == E_SHAPE
    assert f(A, 4, 100, A, A, 0, None) == E_SHAPE
    assert f(A, 4, -128, A, A, 0, None) == E_SHAPE
    assert f(A + 8, 4, 128, A, A, 0, None) == E_ALIGN
    assert f(A, 4, 128, A + 4, A, 0, None) == E_ALIGN
    assert f(A, 4, 128, A, A + 2, 0, None) == E_ALIGN
    assert f(A, 4, 128, A, A, 2, None) == E_ENUM
    assert f(A, 4, 128, A, A, -1, None) == E_ENUM


def test_quantize_weight_validation(lib):
    f = lib.fp8q_quantize_weight
    assert f(None, 128, 128, A, A, 0, None) == E_NULL
    assert f(A, 100, 128, A, A, 0, None) == E_SHAPE
    assert f(A, 128, 130, A, A, 0, None) == E_SHAPE
    assert f(A + 16 + 8, 128, 128, A, A, 0, None) == E_ALIGN
    assert f(A, 128, 128, A, A, 7, None) == E_ENUM
    assert f(None, 0, 0, None, None, 0, None) == OK


def test_debug_checks_flag():
    assert _load(LIB).fp8q_debug_checks() == 0
    assert _load(LIB_DEBUG).fp8q_debug_checks() == 1


@pytest.mark.parametrize("name", ["fp8q_gemm", "fp8q_gemm_precise", "fp8q_gemm_mfma_scaled"])
def test_gemm_validation(lib, name):
    f = getattr(lib, name)
    assert f(A, A, A, A, 4, 128, 128, None, 0, None) == E_NULL
    assert f(None, A, A, A, 4, 128, 128, A, 0, None) == E_NULL
    assert f(A, None, A, A, 4, 128, 128, A, 0, None) == E_NULL
    assert f(A, A, A, A, 4, 100, 128, A, 0, None) == E_SHAPE
    assert f(A, A, A, A, 4, 128, 64, A, 0, None) == E_SHAPE
    assert f(A, A, A, A, -4, 128, 128, A, 0, None) == E_SHAPE
    assert f(A, A, A + 1, A, 4, 128, 128, A, 0, None) == E_ALIGN
    assert f(A, A + 1, A, A, 4, 128, 128, A, 0, None) == E_ALIGN
    assert f(A, A, A, A, 4, 128, 128, A + 8, 0, None) == E_ALIGN
    assert f(A, A, A, A, 4, 128, 128, A, 3, None) == E_ENUM
    assert f(None, None, None, None, 0, 128, 128, None, 0, None) == OK
    # valid requests outside the library's range (host-side, before any device call)
    assert f(A, A, A, A, 4, 128, 0, A, 0, None) == E_UNSUP            # K == 0: C = 0
    assert f(A, A, A, A, 4, 128, (1 << 22) + 128, A, 0, None) == E_UNSUP
    assert f(A, A, A, A, 1 << 29, 128, 128, A, 0, None) == E_UNSUP    # scale offsets >= 2^31


@pytest.mark.parametrize("name", ["fp8q_grouped_gemm", "fp8q_grouped_gemm_precise"])
def test_grouped_gemm_validation(lib, name):
    f = getattr(lib, name)
    assert f(A, A, 8, None, 2, A, A, 128, 128, A, 0, None) == E_NULL
    assert f(A, A, 8, A, 2, A, A, 128, 128, None, 0, None) == E_NULL
    assert f(A, A, 8, A, 0, A, A, 128, 128, A, 0, None) == E_SHAPE
    assert f(A, A, 8, A, 2, A, A, 200, 128, A, 0, None) == E_SHAPE
    assert f(A, A, -8, A, 2, A, A, 128, 128, A, 0, None) == E_SHAPE
    assert f(A, A, 8, A + 2, 2, A, A, 128, 128, A, 0, None) == E_ALIGN
    assert f(A, A, 8, A, 2, A, A, 128, 128, A, 5, None) == E_ENUM
    assert f(A, A, 8, A, 2000, A, A, 128, 128, A, 0, None) == E_UNSUP
    assert f(A, A, 8, A, 2, A, A, 128, 0, A, 0, None) == E_UNSUP
    assert f(A, A, 8, A, 2, A, A, 128, (1 << 22) + 128, A, 0, None) == E_UNSUP
    assert f(None, None, 0, A, 2, None, None, 128, 128, None, 0, None) == OK


def test_gemm_bf16_validation(lib):
    f = lib.fp8q_gemm_bf16
    assert f(A, A, 4, 128, 128, None, 0, None) == E_NULL
    assert f(None, A, 4, 128, 128, A, 0, None) == E_NULL
    assert f(A, None, 4, 128, 128, A, 0, None) == E_NULL
    assert f(A, A, 4, 100, 128, A, 0, None) == E_SHAPE
    assert f(A, A, 4, 128, 64, A, 0, None) == E_SHAPE
    assert f(A, A, -4, 128, 128, A, 0, None) == E_SHAPE
    assert f(A + 2, A, 4, 128, 128, A, 0, None) == E_ALIGN
    assert f(A, A + 8, 4, 128, 128, A, 0, None) == E_ALIGN
    assert f(A, A, 4, 128, 128, A + 4, 0, None) == E_ALIGN
    assert f(A, A, 4, 128, 128, A, 2, None) == E_ENUM
    assert f(None, None, 0, 128, 128, None, 0, None) == OK
    assert f(A, A, 4, 128, 0, A, 0, None) == E_UNSUP                  # K == 0: C = 0
    assert f(A, A, 4, 128, (1 << 21) + 128, A, 0, None) == E_UNSUP    # 2K-byte rows


def test_transposed_quantizer_validation(lib):
    for f in (lib.fp8q_quantize_act_t, lib.fp8q_quantize_weight_t):
        assert f(None, 128, 128, A, A, 0, None) == E_NULL
        assert f(A, 128, 128, None, A, 0, None) == E_NULL
        assert f(A, 128, 128, A, None, 0, None) == E_NULL
        assert f(None, 0, 128, None, None, 0, None) == OK
        assert f(A, 100, 128, A, A, 0, None) == E_SHAPE   # M (or N) must be a multiple of 128
        assert f(A, 128, 64, A, A, 0, None) == E_SHAPE
        assert f(A, -128, 128, A, A, 0, None) == E_SHAPE
        assert f(A + 8, 128, 128, A, A, 0, None) == E_ALIGN
        assert f(A, 128, 128, A + 4, A, 0, None) == E_ALIGN
        assert f(A, 128, 128, A, A + 2, 0, None) == E_ALIGN
        assert f(A, 128, 128, A, A, 2, None) == E_ENUM


@pytest.mark.parametrize("name", ["fp8q_gemm_rowscaled", "fp8q_gemm_rowscaled_precise"])
def test_gemm_rowscaled_validation(lib, name):
    f = getattr(lib, name)
    assert f(A, A, A, A, 4, 128, 128, None, 0, None) == E_NULL
    assert f(A, A, None, A, 4, 128, 128, A, 0, None) == E_NULL
    assert f(A, A, A, None, 4, 128, 128, A, 0, None) == E_NULL
    assert f(A, A, A, A, 4, 100, 128, A, 0, None) == E_SHAPE
    assert f(A, A, A, A, 4, 128, 64, A, 0, None) == E_SHAPE
    assert f(A, A, A + 1, A, 4, 128, 128, A, 0, None) == E_ALIGN
    assert f(A, A, A, A + 2, 4, 128, 128, A, 0, None) == E_ALIGN
    assert f(A, A, A, A, 4, 128, 128, A, 3, None) == E_ENUM
    assert f(None, None, None, None, 0, 128, 128, None, 0, None) == OK
    assert f(A, A, A, A, 4, 128, 0, A, 0, None) == E_UNSUP
    assert f(A, A, A, A, 4, 1 << 29, 128, A, 0, None) == E_UNSUP    # b_s offsets >= 2^31


def test_gemm_fused_validation(lib):
    f = lib.fp8q_gemm_fused
    assert f(A, A, A, 4, 128, 128, None, 0, 0, None) == E_NULL
    assert f(None, A, A, 4, 128, 128, A, 0, 0, None) == E_NULL
    assert f(A, None, A, 4, 128, 128, A, 0, 0, None) == E_NULL
    assert f(A, A, None, 4, 128, 128, A, 0, 0, None) == E_NULL
    assert f(A, A, A, 4, 100, 128, A, 0, 0, None) == E_SHAPE
    assert f(A, A, A, 4, 128, 64, A, 0, 0, None) == E_SHAPE
    assert f(A, A, A, -4, 128, 128, A, 0, 0, None) == E_SHAPE
    assert f(A + 2, A, A, 4, 128, 128, A, 0, 0, None) == E_ALIGN
    assert f(A, A + 8, A, 4, 128, 128, A, 0, 0, None) == E_ALIGN
    assert f(A, A, A + 2, 4, 128, 128, A, 0, 0, None) == E_ALIGN
    assert f(A, A, A, 4, 128, 128, A + 4, 0, 0, None) == E_ALIGN
    assert f(A, A, A, 4, 128, 128, A, 2, 0, None) == E_ENUM       # out dtype
    assert f(A, A, A, 4, 128, 128, A, 0, 2, None) == E_ENUM       # scale mode
    assert f(None, None, None, 0, 128, 128, None, 0, 0, None) == OK
    assert f(A, A, A, 4, 128, 0, A, 0, 0, None) == E_UNSUP
    assert f(A, A, A, 4, 128, (1 << 21) + 128, A, 0, 0, None) == E_UNSUP


def test_grouped_gemm_fused_validation(lib):
    f = lib.fp8q_grouped_gemm_fused
    assert f(A, 8, None, 2, A, A, 128, 128, A, 0, 0, None) == E_NULL
    assert f(A, 8, A, 2, A, A, 128, 128, None, 0, 0, None) == E_NULL
    assert f(None, 8, A, 2, A, A, 128, 128, A, 0, 0, None) == E_NULL
    assert f(A, 8, A, 0, A, A, 128, 128, A, 0, 0, None) == E_SHAPE
    assert f(A, 8, A, 2, A, A, 200, 128, A, 0, 0, None) == E_SHAPE
    assert f(A, -8, A, 2, A, A, 128, 128, A, 0, 0, None) == E_SHAPE
    assert f(A, 8, A + 2, 2, A, A, 128, 128, A, 0, 0, None) == E_ALIGN
    assert f(A + 8, 8, A, 2, A, A, 128, 128, A, 0, 0, None) == E_ALIGN
    assert f(A, 8, A, 2, A, A, 128, 128, A, 5, 0, None) == E_ENUM
    assert f(A, 8, A, 2, A, A, 128, 128, A, 0, 7, None) == E_ENUM
    assert f(A, 8, A, 2000, A, A, 128, 128, A, 0, 0, None) == E_UNSUP
    assert f(A, 8, A, 2, A, A, 128, 0, A, 0, 0, None) == E_UNSUP
    assert f(A, 8, A, 2, A, A, 128, (1 << 21) + 128, A, 0, 0, None) == E_UNSUP
    assert f(None, 0, A, 2, None, None, 128, 128, None, 0, 0, None) == OK


def test_valid_arguments_without_gpu_report_device_error(lib):
    if not _no_device():
        pytest.skip("a GPU is visible: fake pointers must not be launched")
    assert lib.fp8q_quantize_act(A, 4, 128, A, A, 0, None) == E_DEVICE
    assert lib.fp8q_quantize_weight(A, 128, 128, A, A, 1, None) == E_DEVICE
    assert lib.fp8q_gemm(A, A, A, A, 4, 128, 128, A, 1, None) == E_DEVICE
    assert lib.fp8q_grouped_gemm(A, A, 8, A, 2, A, A, 128, 128, A, 0, None) == E_DEVICE
    assert lib.fp8q_gemm_bf16(A, A, 4, 128, 128, A, 0, None) == E_DEVICE
    assert lib.fp8q_quantize_act_t(A, 128, 128, A, A, 0, None) == E_DEVICE
    assert lib.fp8q_quantize_weight_t(A, 128, 128, A, A, 0, None) == E_DEVICE
    assert lib.fp8q_gemm_rowscaled(A, A, A, A, 4, 128, 128, A, 0, None) == E_DEVICE
    assert lib.fp8q_gemm_fused(A, A, A, 4, 128, 128, A, 0, 1, None) == E_DEVICE
    assert lib.fp8q_grouped_gemm_fused(A, 8, A, 2, A, A, 128, 128, A, 0, 0, None) == E_DEVICE
    assert lib.fp8q_gemm_precise(A, A, A, A, 4, 128, 128, A, 1, None) == E_DEVICE
    assert lib.fp8q_gemm_mfma_scaled(A, A, A, A, 4, 128, 128, A, 1, None) == E_DEVICE
    assert lib.fp8q_grouped_gemm_precise(A, A, 8, A, 2, A, A, 128, 128, A, 0, None) == E_DEVICE
    assert lib.fp8q_gemm_rowscaled_precise(A, A, A, A, 4, 128, 128, A, 0, None) == E_DEVICE


def test_probe_library_exports_and_validation():
    """The measurement probes (streaming ceiling, instruction mix) load and
    reject invalid arguments on the host before any HIP call."""
    path = os.path.join(ROOT, "fine_grained_block_fp8q_amd", "libfp8q_probe.so")
    if not os.path.exists(path):
        pytest.fail("libfp8q_probe.so is not built (python fine_grained_block_fp8q_amd/build.py)")
    L = ctypes.CDLL(path)
    p = ctypes.c_void_p
    L.fp8q_probe_stream.argtypes = [p, p, ctypes.c_int64, ctypes.c_int, p]
    L.fp8q_probe_mix.argtypes = [ctypes.c_int, ctypes.c_int, p, p]
    L.fp8q_probe_ring.argtypes = [p, ctypes.c_int64, p, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, p]
    L.fp8q_probe_ring_split.argtypes = [p, ctypes.c_int64, p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, p]
    L.fp8q_probe_ring_reads.argtypes = L.fp8q_probe_ring_split.argtypes
    for name in ("fp8q_probe_stream", "fp8q_probe_mix", "fp8q_probe_cus", "fp8q_probe_ring",
                 "fp8q_probe_ring_split", "fp8q_probe_ring_reads"):
        assert hasattr(L, name)
    reads = L.fp8q_probe_ring_reads
    assert reads(p(4096), 256, p(8192), 256, 7168, 256, 2, 7, 1, 16, None) == -1  # no such count
    assert reads(p(4096), 256, None, 256, 7168, 256, 2, 24, 1, 16, None) == -1    # no A
    assert reads(p(4096), 100, None, 0, 7168, 0, 2, 24, 1, 16, None) == -1        # w_rows
    split = L.fp8q_probe_ring_split
    assert split(p(4096), 256, None, 256, 7168, 256, 2, 3, 1, 16, None) == -1     # no A
    assert split(p(4096), 256, p(8192), 256, 7168, 0, 2, 3, 1, 16, None) == -1    # ra = 0
    assert split(p(4096), 256, p(8192), 300, 7168, 256, 2, 3, 1, 16, None) == -1  # a_rows
    assert split(p(4096), 256, p(8192), 256, 7168, 256, 3, 3, 1, 16, None) == -1  # no such ring
    assert split(p(4096), 256, p(8192), 256, 7100, 256, 2, 3, 1, 16, None) == -1  # K
    assert L.fp8q_probe_ring(None, 256, None, 0, 7168, 0, 2, 1, 16, None) == -1
    assert L.fp8q_probe_ring(p(4096), 100, None, 0, 7168, 0, 2, 1, 16, None) == -1   # w_rows
    assert L.fp8q_probe_ring(p(4096), 256, None, 128, 7168, 128, 3, 1, 16, None) == -1  # no A
    assert L.fp8q_probe_ring(p(4096), 256, p(8192), 200, 7168, 128, 3, 1, 16, None) == -1
    assert L.fp8q_probe_stream(None, None, 1024, 1, None) == -1
    assert L.fp8q_probe_stream(p(4096), p(8192), 1000, 1, None) == -1   # not a multiple of 16
    assert L.fp8q_probe_stream(p(4096), p(8192), 1024, 3, None) == -1   # ratio
    assert L.fp8q_probe_mix(0, 100, None, None) == -1
    assert L.fp8q_probe_mix(0, 0, p(4096), None) == -1
