"""Host-side checks of the Python binding (no GPU needed): every wrapper
rejects wrong dtypes, layouts, devices and shapes with ValueError before any
C call, and bind() validates once and returns a callable for the same call."""

import unittest.mock as um

import pytest
import torch

fq = pytest.importorskip("fine_grained_block_fp8q_amd")


def _t(shape, dt):
    return torch.empty(shape, dtype=dt)


u8, f32, bf16, i32 = torch.uint8, torch.float32, torch.bfloat16, torch.int32


def _no_c_call(*a, **k):
    raise AssertionError("the C library must not be called")


@pytest.fixture(autouse=True)
def no_stream():
    # the wrappers fetch torch's current stream, which needs a GPU
    with um.patch.object(fq, "_stream", lambda st, d: None):
        yield


def test_gemm_argument_checks():
    M, N, K = 64, 256, 384
    good = dict(a_q=_t((M, K), u8), a_s=_t((K // 128, M), f32), w_q=_t((N, K), u8),
                w_s=_t((N // 128, K // 128), f32), c=_t((M, N), f32))
    bad = [
        dict(c=_t((M, N), torch.float16)),                 # fp16 output would be written as fp32
        dict(a_s=_t((K // 128 + 1, M), f32)),               # scale shape
        dict(w_q=_t((N, K + 128), u8)),                     # K mismatch between operands
        dict(w_s=_t((N // 128, K // 128), torch.float64)),  # scale dtype
        dict(a_q=_t((K, M), u8).t()),                       # not contiguous
        dict(c=_t((M + 1, N), f32)),                        # output shape
    ]
    for fn in (fq.fp8q_gemm, fq.fp8q_gemm_precise):
        for b in bad:
            args = {**good, **b}
            with um.patch.object(fq.lib, "fp8q_gemm", _no_c_call), \
                    um.patch.object(fq.lib, "fp8q_gemm_precise", _no_c_call):
                with pytest.raises(ValueError):
                    fn(**args)


def test_grouped_argument_checks():
    Mt, G, N, K = 100, 3, 256, 256
    good = dict(a_q=_t((Mt, K), u8), a_s=_t((K // 128, Mt), f32), off=_t((G + 1,), i32),
                w_q=_t((G, N, K), u8), w_s=_t((G, N // 128, K // 128), f32), c=_t((Mt, N), bf16))
    for b in (dict(off=_t((G,), i32)), dict(off=_t((G + 1,), torch.int64)),
              dict(w_s=_t((G, N // 128, K // 128 + 1), f32)), dict(c=_t((Mt, N + 128), bf16))):
        for fn in (fq.fp8q_grouped_gemm, fq.fp8q_grouped_gemm_precise):
            with pytest.raises(ValueError):
                fn(**{**good, **b})


def test_quantizer_argument_checks():
    M, K = 32, 256
    x, q, s = _t((M, K), bf16), _t((M, K), u8), _t((K // 128, M), f32)
    for args in ((_t((M, K), f32), q, s), (x, _t((M, K), torch.int8), s), (x, q, _t((M, K // 128), f32)),
                 (_t((M, K + 64), bf16), _t((M, K + 64), u8), s)):
        with pytest.raises(ValueError):
            fq.fp8q_quantize_act(*args)


def test_bind_validates_once_and_returns_the_call():
    M, K = 32, 256
    x, q, s = _t((M, K), bf16), _t((M, K), u8), _t((K // 128, M), f32)
    calls = []
    with um.patch.object(fq.lib, "fp8q_quantize_act", lambda *a: calls.append(a) or 0):
        run = fq.bind(fq.fp8q_quantize_act, x, q, s)
        assert calls == []              # binding makes no C call
        run()
        run()
    assert len(calls) == 2 and calls[0][1] == M and calls[0][2] == K
    with pytest.raises(ValueError):     # the checks still run when binding
        fq.bind(fq.fp8q_quantize_act, x, q, _t((3, M), f32))
    assert not getattr(fq._capture, "on", False)
    with um.patch.object(fq.lib, "fp8q_quantize_act", lambda *a: fq.ERR_SHAPE):
        run = fq.bind(fq.fp8q_quantize_act, x, q, s)
        with pytest.raises(fq.Fp8qError):
            run()


def test_bind_keeps_its_tensors_alive():
    """The bound call's pointers stay valid: the callable holds the tensors,
    which are freed only with it."""
    import gc
    import weakref
    M, K = 32, 256
    x, q, s = _t((M, K), bf16), _t((M, K), u8), _t((K // 128, M), f32)
    refs = [weakref.ref(t) for t in (x, q, s)]
    with um.patch.object(fq.lib, "fp8q_quantize_act", lambda *a: 0):
        run = fq.bind(fq.fp8q_quantize_act, x, q, s)
        del x, q, s
        gc.collect()
        assert all(r() is not None for r in refs)
        run()
    del run
    gc.collect()
    assert all(r() is None for r in refs)
