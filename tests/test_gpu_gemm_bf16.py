"""GPU parity of the BF16 GEMM of the same kernel family (fp8q_gemm_bf16)
against the oracle's BF16 reference (oracle.gemm.gemm_bf16), through the C ABI.

Acceptance: every checked output within 1e-5 * sum_k |a_k||w_k| of the exact
product (+ half a BF16 ulp for BF16 output).  BF16 products are exact in FP32
and the matrix core's BF16 path accumulates them to FP32 accuracy, so unlike
the FP8 path no output may exceed the bound.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import fq, to_dev_bf16
from oracle import gemm as ogemm

pytestmark = pytest.mark.gpu


def _run(A_bits, W_bits, out="f32"):
    f = fq()
    a = to_dev_bf16(A_bits)
    w = to_dev_bf16(W_bits)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = torch.empty((a.shape[0], w.shape[0]), dtype=dt, device=a.device)
    f.fp8q_gemm_bf16(a, w, c)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


def _check(c, A_bits, W_bits, out="f32", what=""):
    ref = ogemm.gemm_bf16(A_bits, W_bits)
    tol = 1e-5 * ogemm.abs_bound_bf16(A_bits, W_bits)
    half = ogemm.bf16_half_ulp(ref) if out == "bf16" else 0.0
    err = np.abs(c - ref)
    bad = err > tol + half
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} outputs out of tolerance, first at "
        f"{tuple(np.argwhere(bad)[0])}: gpu {c[bad][0]!r} ref {ref[bad][0]!r}")
    rel = err / np.where(tol > 0, tol / 1e-5, 1.0)
    return {"max_err_over_abs_sum": float(rel.max())}


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_bf16_gemm_tiny_full(out):
    A, W = workloads.dense_inputs("tiny")
    r = _check(_run(A, W, out), A, W, out, f"tiny {out}")
    print(f"tiny {out}: {r}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 384, 640), (255, 256, 256),
                                   (300, 512, 1152), (513, 640, 384), (64, 128, 2048)])
def test_bf16_gemm_ragged_shapes(M, N, K):
    rng = np.random.default_rng(M * 5 + N * 11 + K)
    A = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = workloads.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    _check(_run(A, W), A, W, what=f"{M}x{N}x{K}")


def test_bf16_gemm_same_sign_and_zero_rows():
    """All-positive operands (no cancellation) and an all-zero row."""
    rng = np.random.default_rng(6)
    M, N, K = 200, 256, 1024
    A = np.abs(rng.standard_normal((M, K))).astype(np.float32)
    A[7, :] = 0
    W = np.abs(rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A, W = workloads.bf16_bits(A), workloads.bf16_bits(W)
    c = _run(A, W)
    assert np.all(c[7] == 0)
    _check(c, A, W, what="same sign")


def test_bf16_gemm_dense_full_size_sampled():
    """The dense 4096 x 4096 x 7168 workload in the bench's launch
    configuration; 48 sampled rows checked against every column."""
    cfg = workloads.WORKLOADS["dense"]
    A, W = workloads.dense_inputs("dense")
    c = _run(A, W)
    rows = np.sort(np.random.default_rng(2).choice(cfg["M"], 46, replace=False))
    rows = np.concatenate([[0], rows, [cfg["M"] - 1]])
    r = _check(c[rows], A[rows], W, what="dense sampled")
    print(f"dense bf16: {r}")


def test_bf16_gemm_determinism():
    A, W = workloads.dense_inputs("tiny")
    c1 = _run(A, W)
    c2 = _run(A, W)
    assert np.array_equal(c1, c2)


def test_fp8_path_error_against_bf16_on_dense_workload():
    """Accuracy of the FP8 path on the dense workload (1% x30 outlier channels),
    against the exact product of its BF16 inputs on 32 sampled rows: the FP8
    GEMM carries the E4M3 quantization error (a few percent, as the oracle's
    outlier study predicts); the BF16 GEMM of the same family only FP32
    rounding.  The pages give no magnitude for this, so only the order is
    asserted."""
    cfg = workloads.WORKLOADS["dense"]
    A, W = workloads.dense_inputs("dense")
    f = fq()
    a, w = to_dev_bf16(A), to_dev_bf16(W)
    aq, as_ = f.quantize_act(a)
    wq, ws = f.quantize_weight(w)
    c8 = f.gemm(aq, as_, wq, ws)
    c16 = torch.empty_like(c8)
    f.fp8q_gemm_bf16(a, w, c16)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(cfg["M"], 32, replace=False))
    ref = ogemm.gemm_bf16(A[rows], W)
    e8 = np.linalg.norm(c8.cpu().numpy()[rows] - ref) / np.linalg.norm(ref)
    e16 = np.linalg.norm(c16.cpu().numpy()[rows] - ref) / np.linalg.norm(ref)
    print(f"relative Frobenius error vs the exact BF16 product: FP8 path {e8:.3e}, BF16 GEMM {e16:.3e}")
    assert e16 < 1e-6 and 1e-3 < e8 < 0.06
