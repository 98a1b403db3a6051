"""Edge cases of the GEMM path at the limits of its contract, on the GPU:

1. The largest K the entry points accept (2^22, 32768 chunks) with FP32
   scales: the quantizers bit-exact, both GEMM modes within their contracts
   on every output.
2. Operand magnitudes far from 1 (activations and weights scaled by powers of
   two from 2^-100 to 2^60), chosen so that every product s_a * s_w of group
   scales stays a normal FP32 number, the range the accuracy clauses of
   include/fp8q.h are stated for: codes and scales bit-exact, both GEMM modes
   within their contracts.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_gemm_bounded, assert_gemm_strict, fq, host, to_dev_bf16
from oracle import quant as oquant

pytestmark = pytest.mark.gpu

FLT_MIN = 2.0 ** -126


def _check_quant(gq, gs, rq, rs, what):
    gq, gs = host(gq), host(gs)
    assert np.array_equal(gq, rq), f"{what}: codes differ"
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), f"{what}: scales differ"


def _scale_products(sa, sw):
    """|s_a * s_w| for every (row, weight block, chunk) in float64."""
    return np.abs(sa.astype(np.float64))[:, :, None] * np.abs(sw.astype(np.float64)).T[:, None, :]


def _quantize_weight_sliced(W, mode, parts=8):
    """oracle.quant.quantize_weight over K slices of whole 128-column blocks
    (blocks are independent, so the result is the same; the slices bound the
    oracle's float64 temporaries)."""
    K = W.shape[1]
    step = K // parts
    assert step % 128 == 0
    out = [oquant.quantize_weight(np.ascontiguousarray(W[:, k:k + step]), mode)
           for k in range(0, K, step)]
    return np.concatenate([q for q, _ in out], axis=1), np.concatenate([s for _, s in out], axis=1)


def test_largest_k():
    """K = 2^22 (the ABI's limit), FP32 scales: 4 activation rows (1% outlier
    channels x30) against one 128-row weight block, every output checked."""
    M, N, K, seed, mode = 4, 128, 1 << 22, 2024, "f32"
    print(f"\nlargest K: generating {M}x{K} and {N}x{K}", flush=True)
    outl = workloads.outlier_channels(K, seed, frac=0.01)
    A = workloads.act_rows(np.arange(M), K, seed, 1.0, outl, 30.0)
    W = workloads.rows_threaded(workloads.weight_rows, np.arange(N), K, seed, 0.02)
    f = fq()
    aq, as_ = f.quantize_act(to_dev_bf16(A), mode)
    wq, ws = f.quantize_weight(to_dev_bf16(W), mode)
    c = f.gemm(aq, as_, wq, ws)
    cp = f.gemm(aq, as_, wq, ws, precise=True)
    torch.cuda.synchronize()
    print("largest K: oracle", flush=True)
    qa, sa = oquant.quantize_act(A, mode)
    _check_quant(aq, as_, qa, sa, "largest K act")
    del A, aq
    qw, sw = _quantize_weight_sliced(W, mode)
    _check_quant(wq, ws, qw, sw, "largest K weight")
    del W, wq
    r = assert_gemm_bounded(host(c).astype(np.float64), qa, sa, qw, sw, what="largest K")
    rp = assert_gemm_strict(host(cp).astype(np.float64), qa, sa, qw, sw,
                            what="largest K precise")
    print(f"largest K: fp8 {r}; precise {rp}")


MAGNITUDES = [(-50, -50), (40, 40), (-50, 40), (-100, 60), (60, -100)]


@pytest.mark.parametrize("mode", ["f32", "pow2"])
@pytest.mark.parametrize("ea,ew", MAGNITUDES)
def test_extreme_magnitudes(ea, ew, mode):
    """A ~ N(0,1) * 2^ea (two outlier channels x50), W ~ N(0,1) * 2^ew."""
    M, N, K = 96, 256, 1024
    rng = np.random.default_rng(7000 + 37 * ea + ew)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, rng.choice(K, 2, replace=False)] *= np.float32(50)
    A = workloads.bf16_bits(np.ldexp(a, ea))
    W = workloads.bf16_bits(np.ldexp(rng.standard_normal((N, K)).astype(np.float32), ew))
    qa, sa = oquant.quantize_act(A, mode)
    qw, sw = oquant.quantize_weight(W, mode)
    prod = _scale_products(sa, sw)
    assert prod.min() >= FLT_MIN and prod.max() * 128 * 448.0 ** 2 < 2.0 ** 120, \
        "the case must keep s_a * s_w and the partials in FP32's normal range"
    f = fq()
    aq, as_ = f.quantize_act(to_dev_bf16(A), mode)
    wq, ws = f.quantize_weight(to_dev_bf16(W), mode)
    _check_quant(aq, as_, qa, sa, f"act 2^{ea} {mode}")
    _check_quant(wq, ws, qw, sw, f"weight 2^{ew} {mode}")
    for out in ("f32", "bf16"):
        dt = torch.float32 if out == "f32" else torch.bfloat16
        c = host(f.gemm(aq, as_, wq, ws, out_dtype=dt).float()).astype(np.float64)
        cp = host(f.gemm(aq, as_, wq, ws, out_dtype=dt, precise=True).float()).astype(np.float64)
        assert_gemm_bounded(c, qa, sa, qw, sw, out=out, what=f"2^{ea} x 2^{ew} {mode} {out}")
        assert_gemm_strict(cp, qa, sa, qw, sw, out=out,
                           what=f"precise 2^{ea} x 2^{ew} {mode} {out}")
