"""fp8q_gemm_mfma_scaled: power-of-two group scales applied by the matrix core
(the block-scaled FP8 MFMA's E8M0 operand scales; the "MMA with group
scaling" of the hardware-suggestion passage of why-be.co.kr as_center post
57820), through the C ABI.

Acceptance: on power-of-two-scaled operands within the RANGE clause of
include/fp8q.h (every s_a * s_w a normal FP32 number), the output is bitwise
equal to fp8q_gemm's on every output (scaling by a power of two commutes with
the matrix core's truncation and with FP32 rounding), and it meets fp8q_gemm's
a-priori bound against the exact oracle.  Cases: the tiny workload in full,
ragged shapes, zero groups, scales below 2^-126 (which E8M0 cannot hold
beside the others, split between the matrix core and the promotion), both
output types, and the dense workload at full size.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_gemm_bounded, fq, host, to_dev_bf16
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


def _both(A_bits, W_bits, out="f32"):
    f = fq()
    aq, as_ = f.quantize_act(to_dev_bf16(A_bits), "pow2")
    wq, ws = f.quantize_weight(to_dev_bf16(W_bits), "pow2")
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = f.gemm(aq, as_, wq, ws, out_dtype=dt)
    cm = f.gemm(aq, as_, wq, ws, out_dtype=dt, mfma_scaled=True)
    torch.cuda.synchronize()
    return c, cm, as_, ws


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _assert_equal(c, cm, what):
    a, b = _bits(c), _bits(cm)
    bad = a != b
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs differ from "
                             f"fp8q_gemm; first at {i}: {c[i].item()!r} vs {cm[i].item()!r}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_tiny_workload_equals_fp8q_gemm(out):
    A, W = workloads.dense_inputs("tiny")
    c, cm, _, _ = _both(A, W, out)
    _assert_equal(c, cm, f"tiny {out}")
    qa, sa = oquant.quantize_act(A, "pow2")
    qw, sw = oquant.quantize_weight(W, "pow2")
    ch = cm.float().cpu().numpy().astype(np.float64)
    r = assert_gemm_bounded(ch, qa, sa, qw, sw, out=out, what=f"mfma-scaled tiny {out}")
    print(f"mfma-scaled tiny {out}: {r}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 384, 640), (255, 256, 256),
                                   (300, 512, 1152), (513, 640, 384)])
def test_ragged_shapes_equal_fp8q_gemm(M, N, K):
    rng = np.random.default_rng(M * 11 + N + K)
    A = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = workloads.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    c, cm, _, _ = _both(A, W)
    _assert_equal(c, cm, f"{M}x{N}x{K}")


def test_zero_groups_and_scales_below_the_e8m0_range():
    """Flushed groups (scale 0) and activation groups of BF16 subnormals, whose
    power-of-two scales (2^-141 .. 2^-135) lie below FP32's normal range; the
    weights are large enough (2^40) that every s_a * s_w stays normal."""
    M, N, K = 64, 256, 512
    rng = np.random.default_rng(77)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:8, :128] = 0.0                                   # flushed groups
    a[8:24, 128:256] = np.ldexp(a[8:24, 128:256], -128)  # BF16 subnormals: s_a < 2^-126
    w = np.ldexp(rng.standard_normal((N, K)).astype(np.float32), 40)
    A, W = workloads.bf16_bits(a), workloads.bf16_bits(w)
    c, cm, as_, ws = _both(A, W)
    sa = host(as_).astype(np.float64)
    sw = host(ws).astype(np.float64)
    assert (sa[1, 8:24] < 2.0 ** -126).all() and (sa[1, 8:24] > 0).all(), \
        "the case must reach scales below 2^-126"
    assert (sa[0, :8] == 0).all(), "the case must hold flushed groups"
    prod = sa[:, :, None] * sw.T[:, None, :]
    assert prod[prod > 0].min() >= 2.0 ** -126
    _assert_equal(c, cm, "zero groups / scales below 2^-126")
    qa, sqa = oquant.quantize_act(A, "pow2")
    qw, sqw = oquant.quantize_weight(W, "pow2")
    assert_gemm_bounded(host(cm).astype(np.float64), qa, sqa, qw, sqw,
                        what="mfma-scaled zero groups / small scales")


def test_dense_workload_full_size_equals_fp8q_gemm():
    """The dense 4096 x 4096 x 7168 workload quantized with power-of-two
    scales, every output."""
    A, W = workloads.dense_inputs("dense")
    c, cm, _, _ = _both(A, W)
    _assert_equal(c, cm, "dense pow2")
