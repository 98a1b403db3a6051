"""Python binding of libfp8q (MI355X / gfx950 fine-grained block-scaled FP8).

Argument marshalling only: each function below has the name of the C entry
point it wraps (include/fp8q.h), takes torch tensors, passes their device
pointers, sizes and the current HIP stream, and raises Fp8qError on a non-OK
status.  Every step of the computation runs in the HIP kernels of
libfp8q.so; there is no fallback path -- importing this package without the
built library raises ImportError.

Before each call the wrappers check on the host what the C ABI cannot see
(raising ValueError): every tensor's dtype, contiguity and device, and that
the operand, scale, offset and output shapes agree with each other.  The C
library then validates sizes, alignment and enums itself.

Allocation helpers (``quantize_act``, ``quantize_weight``, ``gemm``,
``grouped_gemm``, ...) allocate outputs with torch on the input's device and
then call the entry points.
"""

import ctypes
import os
import threading

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
lib.fp8q_gemm_precise.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p]
lib.fp8q_gemm_precise.restype = _st
lib.fp8q_gemm_mfma_scaled.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p]
lib.fp8q_gemm_mfma_scaled.restype = _st
lib.fp8q_grouped_gemm.argtypes = [_p, _p, _i64, _p, _i32, _p, _p, _i64, _i64, _p, _i32, _p]
lib.fp8q_grouped_gemm.restype = _st
lib.fp8q_grouped_gemm_precise.argtypes = [_p, _p, _i64, _p, _i32, _p, _p, _i64, _i64, _p, _i32,
                                          _p]
lib.fp8q_grouped_gemm_precise.restype = _st
lib.fp8q_gemm_bf16.argtypes = [_p, _p, _i64, _i64, _i64, _p, _i32, _p]
lib.fp8q_quantize_act_t.argtypes = [_p, _i64, _i64, _p, _p, _i32, _p]
lib.fp8q_quantize_act_t.restype = _st
lib.fp8q_quantize_weight_t.argtypes = [_p, _i64, _i64, _p, _p, _i32, _p]
lib.fp8q_quantize_weight_t.restype = _st
lib.fp8q_gemm_rowscaled.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p]
lib.fp8q_gemm_rowscaled.restype = _st
lib.fp8q_gemm_rowscaled_precise.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p]
lib.fp8q_gemm_rowscaled_precise.restype = _st
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
lib.fp8q_debug_checks.argtypes = []
lib.fp8q_debug_checks.restype = ctypes.c_int

# enums (include/fp8q.h)
(OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ENUM, ERR_DEVICE, ERR_LAUNCH, ERR_UNSUPPORTED,
 ERR_OFFSETS) = range(9)
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


class _Bound(Exception):
    """Raised inside a wrapper called through bind(): carries the C call."""

    def __init__(self, call):
        super().__init__("bound call")
        self.call = call


_capture = threading.local()


def _invoke(cfunc, args, where):
    if getattr(_capture, "on", False):
        raise _Bound((cfunc, args, where))
    _check(cfunc(*args), where)


def bind(fn, *args, **kwargs):
    """Validate a call once and return a zero-argument callable that repeats
    it: the same C entry point with the same pointers, sizes and stream, and
    none of the per-call host checks (for launch loops whose kernels are
    shorter than those checks).  The callable holds references to the
    arguments, so their tensors stay alive while it exists; they must keep
    their storage (no resize or set_) while it is used.  A non-OK status
    still raises.  Example: run = bind(fp8q_quantize_act, x, q, s); run(); run()."""
    _capture.on = True
    try:
        fn(*args, **kwargs)
    except _Bound as b:
        cfunc, cargs, where = b.call
    else:
        raise TypeError(f"{getattr(fn, '__name__', fn)} is not an entry-point wrapper")
    finally:
        _capture.on = False

    keep = (args, kwargs)   # the pointers in cargs refer to these tensors' storage

    def run():
        st = cfunc(*cargs)
        if st != OK:
            raise Fp8qError(st, where)
    run.args = keep
    return run


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(name):
    import torch
    return {"u8": torch.uint8, "f32": torch.float32, "bf16": torch.bfloat16,
            "i32": torch.int32}[name]


def _req(where, name, t, dtypes, shape, device):
    """Host-side check of one tensor argument: dtype, contiguity, device, shape."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{where}: {name} must be a torch.Tensor")
    allowed = [_dt(d) for d in dtypes]
    if t.dtype not in allowed:
        raise ValueError(f"{where}: {name} has dtype {t.dtype}, expected one of {allowed}")
    if not t.is_contiguous():
        raise ValueError(f"{where}: {name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{where}: {name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dims(where, t, ndim, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dim() != ndim:
        raise ValueError(f"{where}: {name} must be a {ndim}-d torch.Tensor")
    return t.shape


def _mult128(where, **dims):
    for k, v in dims.items():
        if v % GROUP:
            raise ValueError(f"{where}: {k} = {v} is not a multiple of {GROUP}")


def _out_code(where, c):
    import torch
    if c.dtype == torch.bfloat16:
        return OUT_BF16
    if c.dtype == torch.float32:
        return OUT_F32
    raise ValueError(f"{where}: c has dtype {c.dtype}, expected float32 or bfloat16")


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
    w = "fp8q_quantize_act"
    M, K = _dims(w, x, 2, "x")
    _mult128(w, K=K)
    _req(w, "x", x, ["bf16"], (M, K), x.device)
    _req(w, "q", q, ["u8"], (M, K), x.device)
    _req(w, "s", s, ["f32"], (K // GROUP, M), x.device)
    _invoke(lib.fp8q_quantize_act, (_ptr(x), M, K, _ptr(q), _ptr(s), _MODES[mode],
                                 _stream(stream, x.device)), "fp8q_quantize_act")


def fp8q_quantize_weight(w, q, s, mode="f32", stream=None):
    """w: bf16 [N][K] -> q: uint8 [N][K], s: float32 [N/128][K/128] (in place)."""
    wh = "fp8q_quantize_weight"
    N, K = _dims(wh, w, 2, "w")
    _mult128(wh, N=N, K=K)
    _req(wh, "w", w, ["bf16"], (N, K), w.device)
    _req(wh, "q", q, ["u8"], (N, K), w.device)
    _req(wh, "s", s, ["f32"], (N // GROUP, K // GROUP), w.device)
    _invoke(lib.fp8q_quantize_weight, (_ptr(w), N, K, _ptr(q), _ptr(s), _MODES[mode],
                                    _stream(stream, w.device)), "fp8q_quantize_weight")


def _gemm_args(where, a_q, a_s, w_q, w_s, c):
    M, K = _dims(where, a_q, 2, "a_q")
    N, _ = _dims(where, w_q, 2, "w_q")
    _mult128(where, N=N, K=K)
    dev = a_q.device
    _req(where, "a_q", a_q, ["u8"], (M, K), dev)
    _req(where, "a_s", a_s, ["f32"], (K // GROUP, M), dev)
    _req(where, "w_q", w_q, ["u8"], (N, K), dev)
    _req(where, "w_s", w_s, ["f32"], (N // GROUP, K // GROUP), dev)
    _req(where, "c", c, ["f32", "bf16"], (M, N), dev)
    return M, N, K, _out_code(where, c)


def fp8q_gemm(a_q, a_s, w_q, w_s, c, stream=None):
    """c[M][N] (float32 or bfloat16) = block-scaled a_q[M][K] x w_q[N][K]^T."""
    M, N, K, out = _gemm_args("fp8q_gemm", a_q, a_s, w_q, w_s, c)
    _invoke(lib.fp8q_gemm, (_ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), M, N, K, _ptr(c), out,
                         _stream(stream, a_q.device)), "fp8q_gemm")


def fp8q_gemm_precise(a_q, a_s, w_q, w_s, c, stream=None):
    """fp8q_gemm with each chunk partial formed by FP16 MFMAs on the widened codes."""
    M, N, K, out = _gemm_args("fp8q_gemm_precise", a_q, a_s, w_q, w_s, c)
    _invoke(lib.fp8q_gemm_precise, (_ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), M, N, K, _ptr(c),
                                 out, _stream(stream, a_q.device)), "fp8q_gemm_precise")


def fp8q_gemm_mfma_scaled(a_q, a_s, w_q, w_s, c, stream=None):
    """fp8q_gemm with power-of-two scales applied by the matrix core (E8M0)."""
    M, N, K, out = _gemm_args("fp8q_gemm_mfma_scaled", a_q, a_s, w_q, w_s, c)
    _invoke(lib.fp8q_gemm_mfma_scaled, (_ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), M, N, K,
                                     _ptr(c), out, _stream(stream, a_q.device)),
            "fp8q_gemm_mfma_scaled")


def _grouped_args(where, a_q, a_s, off, w_q, w_s, c):
    M_total, K = _dims(where, a_q, 2, "a_q")
    G, N, _ = _dims(where, w_q, 3, "w_q")
    _mult128(where, N=N, K=K)
    dev = a_q.device
    _req(where, "a_q", a_q, ["u8"], (M_total, K), dev)
    _req(where, "a_s", a_s, ["f32"], (K // GROUP, M_total), dev)
    _req(where, "off", off, ["i32"], (G + 1,), dev)
    _req(where, "w_q", w_q, ["u8"], (G, N, K), dev)
    _req(where, "w_s", w_s, ["f32"], (G, N // GROUP, K // GROUP), dev)
    _req(where, "c", c, ["f32", "bf16"], (M_total, N), dev)
    return M_total, G, N, K, _out_code(where, c)


def fp8q_grouped_gemm(a_q, a_s, off, w_q, w_s, c, stream=None):
    """Rows [off[e], off[e+1]) of a_q times expert e's w_q[e]; off is a device int32[G+1]."""
    M_total, G, N, K, out = _grouped_args("fp8q_grouped_gemm", a_q, a_s, off, w_q, w_s, c)
    _invoke(lib.fp8q_grouped_gemm, (_ptr(a_q), _ptr(a_s), M_total, _ptr(off), G, _ptr(w_q),
                                 _ptr(w_s), N, K, _ptr(c), out, _stream(stream, a_q.device)), "fp8q_grouped_gemm")


def fp8q_grouped_gemm_precise(a_q, a_s, off, w_q, w_s, c, stream=None):
    """fp8q_grouped_gemm in the precise mode (FP16 MFMAs on the widened codes)."""
    M_total, G, N, K, out = _grouped_args("fp8q_grouped_gemm_precise", a_q, a_s, off, w_q, w_s,
                                          c)
    _invoke(lib.fp8q_grouped_gemm_precise, (_ptr(a_q), _ptr(a_s), M_total, _ptr(off), G, _ptr(w_q),
                                         _ptr(w_s), N, K, _ptr(c), out,
                                         _stream(stream, a_q.device)), "fp8q_grouped_gemm_precise")


def fp8q_gemm_fused(x, w_q, w_s, c, mode="f32", stream=None):
    """c[M][N] = fp8q_gemm(quantize_act(x, mode), w_q, w_s), x: bf16 [M][K]
    quantized inside the GEMM."""
    wh = "fp8q_gemm_fused"
    M, K = _dims(wh, x, 2, "x")
    N, _ = _dims(wh, w_q, 2, "w_q")
    _mult128(wh, N=N, K=K)
    _req(wh, "x", x, ["bf16"], (M, K), x.device)
    _req(wh, "w_q", w_q, ["u8"], (N, K), x.device)
    _req(wh, "w_s", w_s, ["f32"], (N // GROUP, K // GROUP), x.device)
    _req(wh, "c", c, ["f32", "bf16"], (M, N), x.device)
    out = _out_code(wh, c)
    _invoke(lib.fp8q_gemm_fused, (_ptr(x), _ptr(w_q), _ptr(w_s), M, N, K, _ptr(c), out,
                               _MODES[mode], _stream(stream, x.device)), "fp8q_gemm_fused")


def fp8q_grouped_gemm_fused(x, off, w_q, w_s, c, mode="f32", stream=None):
    """The grouped GEMM of quantize_act(x, mode), x: bf16 [M_total][K]
    quantized inside the GEMM; off is a device int32[G+1]."""
    wh = "fp8q_grouped_gemm_fused"
    M_total, K = _dims(wh, x, 2, "x")
    G, N, _ = _dims(wh, w_q, 3, "w_q")
    _mult128(wh, N=N, K=K)
    _req(wh, "x", x, ["bf16"], (M_total, K), x.device)
    _req(wh, "off", off, ["i32"], (G + 1,), x.device)
    _req(wh, "w_q", w_q, ["u8"], (G, N, K), x.device)
    _req(wh, "w_s", w_s, ["f32"], (G, N // GROUP, K // GROUP), x.device)
    _req(wh, "c", c, ["f32", "bf16"], (M_total, N), x.device)
    out = _out_code(wh, c)
    _invoke(lib.fp8q_grouped_gemm_fused, (_ptr(x), M_total, _ptr(off), G, _ptr(w_q), _ptr(w_s), N,
                                       K, _ptr(c), out, _MODES[mode],
                                       _stream(stream, x.device)), "fp8q_grouped_gemm_fused")


def fp8q_gemm_bf16(a, w, c, stream=None):
    """c[M][N] (float32 or bfloat16) = a[M][K] x w[N][K]^T, BF16 operands."""
    wh = "fp8q_gemm_bf16"
    M, K = _dims(wh, a, 2, "a")
    N, _ = _dims(wh, w, 2, "w")
    _mult128(wh, N=N, K=K)
    _req(wh, "a", a, ["bf16"], (M, K), a.device)
    _req(wh, "w", w, ["bf16"], (N, K), a.device)
    _req(wh, "c", c, ["f32", "bf16"], (M, N), a.device)
    out = _out_code(wh, c)
    _invoke(lib.fp8q_gemm_bf16, (_ptr(a), _ptr(w), M, N, K, _ptr(c), out, _stream(stream, a.device)), "fp8q_gemm_bf16")


def fp8q_quantize_act_t(x, q_t, s_t, mode="f32", stream=None):
    """x: bf16 [M][K] -> q_t: uint8 [K][M], s_t: float32 [M/128][K] (in place)."""
    wh = "fp8q_quantize_act_t"
    M, K = _dims(wh, x, 2, "x")
    _mult128(wh, M=M, K=K)
    _req(wh, "x", x, ["bf16"], (M, K), x.device)
    _req(wh, "q_t", q_t, ["u8"], (K, M), x.device)
    _req(wh, "s_t", s_t, ["f32"], (M // GROUP, K), x.device)
    _invoke(lib.fp8q_quantize_act_t, (_ptr(x), M, K, _ptr(q_t), _ptr(s_t), _MODES[mode],
                                   _stream(stream, x.device)), "fp8q_quantize_act_t")


def fp8q_quantize_weight_t(w, q_t, s_t, mode="f32", stream=None):
    """w: bf16 [N][K] -> q_t: uint8 [K][N], s_t: float32 [K/128][N/128] (in place)."""
    wh = "fp8q_quantize_weight_t"
    N, K = _dims(wh, w, 2, "w")
    _mult128(wh, N=N, K=K)
    _req(wh, "w", w, ["bf16"], (N, K), w.device)
    _req(wh, "q_t", q_t, ["u8"], (K, N), w.device)
    _req(wh, "s_t", s_t, ["f32"], (K // GROUP, N // GROUP), w.device)
    _invoke(lib.fp8q_quantize_weight_t, (_ptr(w), N, K, _ptr(q_t), _ptr(s_t), _MODES[mode],
                                      _stream(stream, w.device)), "fp8q_quantize_weight_t")


def _rowscaled_args(where, a_q, a_s, b_q, b_s, c):
    M, K = _dims(where, a_q, 2, "a_q")
    N, _ = _dims(where, b_q, 2, "b_q")
    _mult128(where, N=N, K=K)
    dev = a_q.device
    _req(where, "a_q", a_q, ["u8"], (M, K), dev)
    _req(where, "a_s", a_s, ["f32"], (K // GROUP, M), dev)
    _req(where, "b_q", b_q, ["u8"], (N, K), dev)
    _req(where, "b_s", b_s, ["f32"], (K // GROUP, N), dev)
    _req(where, "c", c, ["f32", "bf16"], (M, N), dev)
    return M, N, K, _out_code(where, c)


def fp8q_gemm_rowscaled(a_q, a_s, b_q, b_s, c, stream=None):
    """c[M][N] = a_q[M][K] x b_q[N][K]^T with 1x128 row-group scales on both."""
    M, N, K, out = _rowscaled_args("fp8q_gemm_rowscaled", a_q, a_s, b_q, b_s, c)
    _invoke(lib.fp8q_gemm_rowscaled, (_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), M, N, K, _ptr(c),
                                   out, _stream(stream, a_q.device)), "fp8q_gemm_rowscaled")


def fp8q_gemm_rowscaled_precise(a_q, a_s, b_q, b_s, c, stream=None):
    """fp8q_gemm_rowscaled in the precise mode (FP16 MFMAs on the widened codes)."""
    M, N, K, out = _rowscaled_args("fp8q_gemm_rowscaled_precise", a_q, a_s, b_q, b_s, c)
    _invoke(lib.fp8q_gemm_rowscaled_precise, (_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), M, N, K,
                                           _ptr(c), out, _stream(stream, a_q.device)), "fp8q_gemm_rowscaled_precise")


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


def gemm_rowscaled(a_q, a_s, b_q, b_s, out_dtype=None, stream=None, precise=False):
    import torch
    out_dtype = out_dtype or torch.float32
    c = torch.empty((a_q.shape[0], b_q.shape[0]), dtype=out_dtype, device=a_q.device)
    f = fp8q_gemm_rowscaled_precise if precise else fp8q_gemm_rowscaled
    f(a_q, a_s, b_q, b_s, c, stream)
    return c


def gemm(a_q, a_s, w_q, w_s, out_dtype=None, stream=None, precise=False, mfma_scaled=False):
    import torch
    out_dtype = out_dtype or torch.float32
    c = torch.empty((a_q.shape[0], w_q.shape[0]), dtype=out_dtype, device=a_q.device)
    assert not (precise and mfma_scaled), "one GEMM mode"
    f = fp8q_gemm_precise if precise else fp8q_gemm_mfma_scaled if mfma_scaled else fp8q_gemm
    f(a_q, a_s, w_q, w_s, c, stream)
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


def grouped_gemm(a_q, a_s, off, w_q, w_s, out_dtype=None, stream=None, precise=False):
    import torch
    out_dtype = out_dtype or torch.float32
    c = torch.empty((a_q.shape[0], w_q.shape[1]), dtype=out_dtype, device=a_q.device)
    f = fp8q_grouped_gemm_precise if precise else fp8q_grouped_gemm
    f(a_q, a_s, off, w_q, w_s, c, stream)
    return c
