"""GPU parity of the backward GEMMs of a linear layer in FP8 (Dgrad and Wgrad)
through the C ABI: the transposed quantizers bit-exact against the oracle,
and the GEMMs against the exact oracle: the precise calls within 1e-5 *
sum_k |a_k||b_k| on every checked output (gpu_util.assert_gemm_strict), the
FP8-MFMA calls within their truncation bound (gpu_util.assert_gemm_bounded).

For Y = X W^T:  dX = dY W   = fp8q_gemm(quantize_act(dY), quantize_weight_t(W))
                dW = dY^T X = fp8q_gemm_rowscaled(quantize_act_t(dY), quantize_act_t(X))
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_gemm_bounded, assert_gemm_strict, fq, host, to_dev_bf16
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


def _bits(x):
    return workloads.bf16_bits(np.asarray(x, dtype=np.float32))


def _special(M, K, seed):
    """N(0,1) with an x40 outlier column, a flushed (all-zero) 128-row group of
    one column, a column of BF16 subnormals and mixed-sign tiny values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, 3] *= 40
    x[:128, 7] = 0
    x[:, 9] = np.float32(2.0 ** -130) * rng.integers(-3, 4, size=M)
    x[:, 11] *= 1e-30
    return _bits(x)


def _same(gpu_q, gpu_s, q, s):
    assert np.array_equal(host(gpu_q), q)
    assert np.array_equal(host(gpu_s).view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("M,K,mode", [(128, 128, "f32"), (256, 384, "f32"), (384, 1152, "f32"),
                                      (256, 384, "pow2"), (1024, 256, "f32")])
def test_quantize_act_t_bit_exact(M, K, mode):
    X = _special(M, K, M + K)
    q, s = fq().quantize_act_t(to_dev_bf16(X), mode)
    torch.cuda.synchronize()
    _same(q, s, *oquant.quantize_act_t(X, mode))


@pytest.mark.parametrize("N,K,mode", [(128, 128, "f32"), (384, 256, "f32"), (256, 640, "pow2")])
def test_quantize_weight_t_bit_exact(N, K, mode):
    W = _special(N, K, 3 * N + K)
    w = to_dev_bf16(W)
    q, s = fq().quantize_weight_t(w, mode)
    q2, s2 = fq().quantize_weight(w, mode)
    torch.cuda.synchronize()
    _same(q, s, *oquant.quantize_weight_t(W, mode))
    # the same blocks as the forward quantizer, transposed
    assert torch.equal(q, q2.t().contiguous()) and torch.equal(s, s2.t().contiguous())


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 384, 640), (300, 512, 1152),
                                   (513, 256, 384), (256, 256, 2048)])
def test_gemm_rowscaled_parity(M, N, K):
    rng = np.random.default_rng(M * 13 + N + K)
    A = _bits(rng.standard_normal((M, K)))
    B = _bits(rng.standard_normal((N, K)) * np.exp2(rng.integers(-4, 5, size=(N, 1))))
    f = fq()
    qa, sa = f.quantize_act(to_dev_bf16(A))
    qb, sb = f.quantize_act(to_dev_bf16(B))
    c = f.gemm_rowscaled(qa, sa, qb, sb)
    cp = f.gemm_rowscaled(qa, sa, qb, sb, precise=True)
    torch.cuda.synchronize()
    oa, osa = oquant.quantize_act(A)
    ob, osb = oquant.quantize_act(B)
    assert_gemm_bounded(host(c), oa, osa, ob, osb, what=f"rowscaled {M}x{N}x{K}",
                        rowscaled=True)
    assert_gemm_strict(host(cp), oa, osa, ob, osb, what=f"rowscaled precise {M}x{N}x{K}",
                       rowscaled=True)


def test_gemm_rowscaled_both_tile_widths():
    """The launcher picks 256 x 224 tiles when they fill the CUs' rounds
    better, else 256 x 256: on 256 CUs a 4096 x 4096 output is one round of
    256 tiles of 256 x 256 (two of 224), and 4096 x 7168 two rounds either
    way.  Both outputs are checked on sampled rows, and the narrower tiles'
    ragged last column tile (7168 = 32 x 224; 4096 = 18 x 224 + 64) too."""
    rng = np.random.default_rng(31)
    f = fq()
    for M, N, K in [(4096, 4096, 256), (4096, 7168, 256), (512, 4096, 384)]:
        A = _bits(rng.standard_normal((M, K)))
        B = _bits(rng.standard_normal((N, K)))
        qa, sa = f.quantize_act(to_dev_bf16(A))
        qb, sb = f.quantize_act(to_dev_bf16(B))
        c = f.gemm_rowscaled(qa, sa, qb, sb)
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(M + N).choice(M, 8, replace=False))
        oa, osa = oquant.quantize_act(A[rows])
        ob, osb = oquant.quantize_act(B)
        assert_gemm_bounded(host(c)[rows], oa, osa, ob, osb, rowscaled=True,
                            bound_cols=np.arange(0, N, 7), what=f"rowscaled {M}x{N}x{K}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_backward_of_a_linear_layer(out):
    """Dgrad and Wgrad of Y = X W^T, each composed from the entry points, against
    the oracle composed the same way (codes bit-exact, GEMMs to the parity bar)."""
    rng = np.random.default_rng(21)
    M, N, K = 512, 640, 768
    X = workloads.act_rows(np.arange(M), K, 21, 1.0,
                           workloads.outlier_channels(K, 21, 0.01, None), 30.0)
    W = _bits(rng.standard_normal((N, K)) * 0.02)
    dY = _bits(rng.standard_normal((M, N)) * 1e-2)
    f = fq()
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    x, w, dy = to_dev_bf16(X), to_dev_bf16(W), to_dev_bf16(dY)
    qd, sd = f.quantize_act(dy)
    qwt, swt = f.quantize_weight_t(w)
    dX = f.gemm(qd, sd, qwt, swt, out_dtype=dt)
    dXp = f.gemm(qd, sd, qwt, swt, out_dtype=dt, precise=True)
    qdt, sdt = f.quantize_act_t(dy)
    qxt, sxt = f.quantize_act_t(x)
    dW = f.gemm_rowscaled(qdt, sdt, qxt, sxt, out_dtype=dt)
    dWp = f.gemm_rowscaled(qdt, sdt, qxt, sxt, out_dtype=dt, precise=True)
    torch.cuda.synchronize()
    od = oquant.quantize_act(dY)
    owt = oquant.quantize_weight_t(W)
    odt = oquant.quantize_act_t(dY)
    oxt = oquant.quantize_act_t(X)
    _same(qwt, swt, *owt)
    _same(qdt, sdt, *odt)
    _same(qxt, sxt, *oxt)
    r1 = assert_gemm_bounded(dX.float().cpu().numpy(), *od, *owt, out=out, what="dgrad")
    r2 = assert_gemm_bounded(dW.float().cpu().numpy(), *odt, *oxt, out=out, what="wgrad",
                             rowscaled=True)
    r3 = assert_gemm_strict(dXp.float().cpu().numpy(), *od, *owt, out=out, what="dgrad precise")
    r4 = assert_gemm_strict(dWp.float().cpu().numpy(), *odt, *oxt, out=out,
                            what="wgrad precise", rowscaled=True)
    print(f"dgrad {r1}\nwgrad {r2}\ndgrad precise {r3}\nwgrad precise {r4}")


def test_wgrad_dense_shape_sampled():
    """Wgrad at the dense workload's shape: 4096 tokens of X (4096 x 7168, the
    dense activation recipe) and dY (4096 x 4096), dW = dY^T X (4096 x 7168,
    inner dimension 4096); 12 sampled rows of dW against every column."""
    c = workloads.WORKLOADS["dense"]
    M, N, K = c["M"], c["N"], c["K"]
    outl = workloads.outlier_channels(K, c["seed"], c["outlier_frac"], c["outlier_count"])
    X = workloads.act_rows(np.arange(M), K, c["seed"], c["act_std"], outl, c["outlier_mult"])
    dY = _bits(np.random.default_rng(22).standard_normal((M, N)) * 1e-2)
    f = fq()
    qdt, sdt = f.quantize_act_t(to_dev_bf16(dY))
    qxt, sxt = f.quantize_act_t(to_dev_bf16(X))
    dW = f.gemm_rowscaled(qdt, sdt, qxt, sxt)
    dWp = f.gemm_rowscaled(qdt, sdt, qxt, sxt, precise=True)
    torch.cuda.synchronize()
    odt = oquant.quantize_act_t(dY)
    oxt = oquant.quantize_act_t(X)
    _same(qdt, sdt, *odt)
    _same(qxt, sxt, *oxt)
    rows = np.sort(np.random.default_rng(23).choice(N, 10, replace=False))
    rows = np.concatenate([[0], rows, [N - 1]])
    r = assert_gemm_bounded(host(dW)[rows], odt[0][rows], odt[1][:, rows], *oxt,
                            what="wgrad dense shape", rowscaled=True,
                            bound_cols=np.arange(0, K, 13))
    rp = assert_gemm_strict(host(dWp)[rows], odt[0][rows], odt[1][:, rows], *oxt,
                            what="wgrad precise dense shape", rowscaled=True)
    print(f"wgrad dense shape: fp8 {r}; precise {rp}")
