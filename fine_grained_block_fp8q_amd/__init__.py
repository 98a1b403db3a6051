"""Python binding of libfp8q (MI355X / gfx950 fine-grained block-scaled FP8).

Argument marshalling only: each function below has the name of the C entry
point it wraps (include/fp8q.h), takes torch tensors, passes their device
pointers, sizes and the current HIP stream, and raises Fp8qError on a non-OK
status.  Every step of the computation runs in the HIP kernels of
libfp8q.so; there is no fallback path -- importing this package without the
built library raises ImportError.

Allocation helpers (``quantize_act``, ``quantize_weight``, ``gemm``,
``grouped_gemm``) allocate outputs with torch on the input's device and then
call the entry points.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8q.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libfp8q.so not found at {LIB_PATH}; build it with "
        "`python fine_grained_block_fp8q_amd/build.py` (hipcc, gfx950)")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_st = ctypes.c_int

lib.fp8q_quantize_act.argtypes = [_p, _i64, _i64, _p, _p, _i32, _p]
lib.fp8q_quantize_act.restype = _st
lib.fp8q_quantize_weight.argtypes = [_p, _i64, _i64, _p, _p, _i32, _p]
lib.fp8q_quantize_weight.restype = _st
lib.fp8q_gemm.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p]
lib.fp8q_gemm.restype = _st
lib.fp8q_grouped_gemm.argtypes = [_p, _p, _i64, _p, _i32, _p, _p, _i64, _i64, _p, _i32, _p]
lib.fp8q_grouped_gemm.restype = _st
lib.fp8q_gemm_bf16.argtypes = [_p, _p, _i64, _i64, _i64, _p, _i32, _p]
lib.fp8q_quantize_act_t.argtypes = [_p, _i64, _i64, _p, _p, _i32, _p]
lib.fp8q_quantize_act_t.restype = _st
lib.fp8q_quantize_weight_t.argtypes = [_p, _i64, _i64, _p, _p, _i32, _p]
lib.fp8q_quantize_weight_t.restype = _st
lib.fp8q_gemm_rowscaled.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p]
lib.fp8q_gemm_rowscaled.restype = _st
lib.fp8q_gemm_bf16.restype = _st
lib.fp8q_gemm_fused.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _i32, _i32, _p]
lib.fp8q_gemm_fused.restype = _st
lib.fp8q_grouped_gemm_fused.argtypes = [_p, _i64, _p, _i32, _p, _p, _i64, _i64, _p, _i32, _i32,
                                        _p]
lib.fp8q_grouped_gemm_fused.restype = _st
lib.fp8q_status_string.argtypes = [_st]
lib.fp8q_status_string.restype = ctypes.c_char_p
lib.fp8q_abi_version.argtypes = []
lib.fp8q_abi_version.restype = ctypes.c_int

# enums (include/fp8q.h)
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ENUM, ERR_DEVICE, ERR_LAUNCH, ERR_UNSUPPORTED = range(8)
SCALE_F32, SCALE_POW2 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
GROUP = 128

_MODES = {"f32": SCALE_F32, "pow2": SCALE_POW2, SCALE_F32: SCALE_F32, SCALE_POW2: SCALE_POW2}
_OUTS = {"f32": OUT_F32, "bf16": OUT_BF16, OUT_F32: OUT_F32, OUT_BF16: OUT_BF16}


class Fp8qError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {lib.fp8q_status_string(status).decode()}")


def _check(status, where):
    if status != OK:
        raise Fp8qError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def abi_version():
    return lib.fp8q_abi_version()


# ---------------------------------------------------------------- entry points
def fp8q_quantize_act(x, q, s, mode="f32", stream=None):
    """x: bf16 [M][K] -> q: uint8 [M][K], s: float32 [K/128][M] (in place)."""
    M, K = x.shape
    _check(lib.fp8q_quantize_act(_ptr(x), M, K, _ptr(q), _ptr(s), _MODES[mode],
                                 _stream(stream, x.device)), "fp8q_quantize_act")


def fp8q_quantize_weight(w, q, s, mode="f32", stream=None):
    """w: bf16 [N][K] -> q: uint8 [N][K], s: float32 [N/128][K/128] (in place)."""
    N, K = w.shape
    _check(lib.fp8q_quantize_weight(_ptr(w), N, K, _ptr(q), _ptr(s), _MODES[mode],
                                    _stream(stream, w.device)), "fp8q_quantize_weight")


def fp8q_gemm(a_q, a_s, w_q, w_s, c, stream=None):
    """c[M][N] (float32 or bfloat16) = block-scaled a_q[M][K] x w_q[N][K]^T."""
    import torch
    M, K = a_q.shape
    N = w_q.shape[0]
    out = OUT_BF16 if c.dtype == torch.bfloat16 else OUT_F32
    _check(lib.fp8q_gemm(_ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), M, N, K, _ptr(c), out,
                         _stream(stream, a_q.device)), "fp8q_gemm")


def fp8q_grouped_gemm(a_q, a_s, off, w_q, w_s, c, stream=None):
    """Rows [off[e], off[e+1]) of a_q times expert e's w_q[e]; off is a device int32[G+1]."""
    import torch
    M_total, K = a_q.shape
    G, N, _ = w_q.shape
    out = OUT_BF16 if c.dtype == torch.bfloat16 else OUT_F32
    _check(lib.fp8q_grouped_gemm(_ptr(a_q), _ptr(a_s), M_total, _ptr(off), G, _ptr(w_q),
                                 _ptr(w_s), N, K, _ptr(c), out, _stream(stream, a_q.device)),
           "fp8q_grouped_gemm")


def fp8q_gemm_fused(x, w_q, w_s, c, mode="f32", stream=None):
    """c[M][N] = fp8q_gemm(quantize_act(x, mode), w_q, w_s), x: bf16 [M][K]
    quantized inside the GEMM."""
    import torch
    M, K = x.shape
    N = w_q.shape[0]
    out = OUT_BF16 if c.dtype == torch.bfloat16 else OUT_F32
    _check(lib.fp8q_gemm_fused(_ptr(x), _ptr(w_q), _ptr(w_s), M, N, K, _ptr(c), out,
                               _MODES[mode], _stream(stream, x.device)), "fp8q_gemm_fused")


def fp8q_grouped_gemm_fused(x, off, w_q, w_s, c, mode="f32", stream=None):
    """The grouped GEMM of quantize_act(x, mode), x: bf16 [M_total][K]
    quantized inside the GEMM; off is a device int32[G+1]."""
    import torch
    M_total, K = x.shape
    G, N, _ = w_q.shape
    out = OUT_BF16 if c.dtype == torch.bfloat16 else OUT_F32
    _check(lib.fp8q_grouped_gemm_fused(_ptr(x), M_total, _ptr(off), G, _ptr(w_q), _ptr(w_s), N,
                                       K, _ptr(c), out, _MODES[mode],
                                       _stream(stream, x.device)),
           "fp8q_grouped_gemm_fused")


def fp8q_gemm_bf16(a, w, c, stream=None):
    """c[M][N] (float32 or bfloat16) = a[M][K] x w[N][K]^T, BF16 operands."""
    import torch
    M, K = a.shape
    N = w.shape[0]
    out = OUT_BF16 if c.dtype == torch.bfloat16 else OUT_F32
    _check(lib.fp8q_gemm_bf16(_ptr(a), _ptr(w), M, N, K, _ptr(c), out, _stream(stream, a.device)),
           "fp8q_gemm_bf16")


def fp8q_quantize_act_t(x, q_t, s_t, mode="f32", stream=None):
    """x: bf16 [M][K] -> q_t: uint8 [K][M], s_t: float32 [M/128][K] (in place)."""
    M, K = x.shape
    _check(lib.fp8q_quantize_act_t(_ptr(x), M, K, _ptr(q_t), _ptr(s_t), _MODES[mode],
                                   _stream(stream, x.device)), "fp8q_quantize_act_t")


def fp8q_quantize_weight_t(w, q_t, s_t, mode="f32", stream=None):
    """w: bf16 [N][K] -> q_t: uint8 [K][N], s_t: float32 [K/128][N/128] (in place)."""
    N, K = w.shape
    _check(lib.fp8q_quantize_weight_t(_ptr(w), N, K, _ptr(q_t), _ptr(s_t), _MODES[mode],
                                      _stream(stream, w.device)), "fp8q_quantize_weight_t")


def fp8q_gemm_rowscaled(a_q, a_s, b_q, b_s, c, stream=None):
    """c[M][N] = a_q[M][K] x b_q[N][K]^T with 1x128 row-group scales on both."""
    import torch
    M, K = a_q.shape
    N = b_q.shape[0]
    out = OUT_BF16 if c.dtype == torch.bfloat16 else OUT_F32
    _check(lib.fp8q_gemm_rowscaled(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), M, N, K, _ptr(c),
                                   out, _stream(stream, a_q.device)), "fp8q_gemm_rowscaled")


# ---------------------------------------------------------- allocation helpers
def quantize_act(x, mode="f32", stream=None):
    import torch
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((K // GROUP, M), dtype=torch.float32, device=x.device)
    fp8q_quantize_act(x, q, s, mode, stream)
    return q, s


def quantize_weight(w, mode="f32", stream=None):
    import torch
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N // GROUP, K // GROUP), dtype=torch.float32, device=w.device)
    fp8q_quantize_weight(w, q, s, mode, stream)
    return q, s


def quantize_act_t(x, mode="f32", stream=None):
    import torch
    M, K = x.shape
    q = torch.empty((K, M), dtype=torch.uint8, device=x.device)
    s = torch.empty((M // GROUP, K), dtype=torch.float32, device=x.device)
    fp8q_quantize_act_t(x, q, s, mode, stream)
    return q, s


def quantize_weight_t(w, mode="f32", stream=None):
    import torch
    N, K = w.shape
    q = torch.empty((K, N), dtype=torch.uint8, device=w.device)
    s = torch.empty((K // GROUP, N // GROUP), dtype=torch.float32, device=w.device)
    fp8q_quantize_weight_t(w, q, s, mode, stream)
    return q, s


def gemm_rowscaled(a_q, a_s, b_q, b_s, out_dtype=None, stream=None):
    import torch
    out_dtype = out_dtype or torch.float32
    c = torch.empty((a_q.shape[0], b_q.shape[0]), dtype=out_dtype, device=a_q.device)
    fp8q_gemm_rowscaled(a_q, a_s, b_q, b_s, c, stream)
    return c


def gemm(a_q, a_s, w_q, w_s, out_dtype=None, stream=None):
    import torch
    out_dtype = out_dtype or torch.float32
    c = torch.empty((a_q.shape[0], w_q.shape[0]), dtype=out_dtype, device=a_q.device)
    fp8q_gemm(a_q, a_s, w_q, w_s, c, stream)
    return c


def gemm_fused(x, w_q, w_s, mode="f32", out_dtype=None, stream=None):
    import torch
    out_dtype = out_dtype or torch.float32
    c = torch.empty((x.shape[0], w_q.shape[0]), dtype=out_dtype, device=x.device)
    fp8q_gemm_fused(x, w_q, w_s, c, mode, stream)
    return c


def grouped_gemm_fused(x, off, w_q, w_s, mode="f32", out_dtype=None, stream=None):
    import torch
    out_dtype = out_dtype or torch.float32
    c = torch.empty((x.shape[0], w_q.shape[1]), dtype=out_dtype, device=x.device)
    fp8q_grouped_gemm_fused(x, off, w_q, w_s, c, mode, stream)
    return c


def grouped_gemm(a_q, a_s, off, w_q, w_s, out_dtype=None, stream=None):
    import torch
    out_dtype = out_dtype or torch.float32
    c = torch.empty((a_q.shape[0], w_q.shape[1]), dtype=out_dtype, device=a_q.device)
    fp8q_grouped_gemm(a_q, a_s, off, w_q, w_s, c, stream)
    return c
