"""Every output of the dense and decode workloads at full size, and of the
dense layer's two backward GEMMs, against the exact oracle, through the C ABI.

- The quantizers' codes and scales are bit-exact on every row of the
  workloads' activations and weights.
- The precise calls (fp8q_gemm_precise, fp8q_grouped_gemm_precise) are
  within the stated tolerance 1e-5 * sum|a||b| (and their own (G + 34) u
  bound) on all 4096 x 4096 dense outputs and on every row of every decode
  expert, 4096 columns each.
- The FP8-MFMA calls (fp8q_gemm, fp8q_grouped_gemm) are within their
  a-priori bound T + (G + 20) u sum|a||b| on the same outputs, T evaluated
  by the oracle's C loop (truncation_bound.c) over every product; the
  fraction within 1e-5 * sum|a||b| is reported.

The oracle's exact GEMM and sum|a||b| at these sizes are about 0.5 TFLOP of
float64 work on the host, and T some 10^11 products: tens of seconds.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import (DEV, assert_gemm_bounded, assert_gemm_strict, bf16_to_bits, fq, host,
                      to_dev_bf16)
from oracle import gemm as ogemm
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_dense_workload_every_output():
    A, W = workloads.dense_inputs("dense")
    print(f"\ndense {A.shape[0]}x{W.shape[0]}x{A.shape[1]}", flush=True)
    f = fq()
    aq, as_ = f.quantize_act(to_dev_bf16(A))
    wq, ws = f.quantize_weight(to_dev_bf16(W))
    cp = f.gemm(aq, as_, wq, ws, precise=True)
    c = f.gemm(aq, as_, wq, ws)
    torch.cuda.synchronize()
    qa, sa = oquant.quantize_act(A)
    qw, sw = oquant.quantize_weight(W)
    assert np.array_equal(host(aq), qa), "activation codes"
    assert np.array_equal(host(as_).view(np.uint32), sa.view(np.uint32)), "activation scales"
    assert np.array_equal(host(wq), qw), "weight codes"
    assert np.array_equal(host(ws).view(np.uint32), sw.view(np.uint32)), "weight scales"
    ref = ogemm.gemm(qa, sa, qw, sw)
    absb = ogemm.abs_bound(qa, sa, qw, sw)
    r = assert_gemm_strict(_f64(cp), qa, sa, qw, sw, what="dense precise, every output",
                           ref=ref, absb=absb)
    rf = assert_gemm_bounded(_f64(c), qa, sa, qw, sw, what="dense fast path, every output",
                             ref=ref, absb=absb, native=True)
    print(f"dense precise: {r}; fast path: {rf}")


def test_decode_workload_every_output():
    cfg = workloads.WORKLOADS["decode"]
    counts, off = workloads.decode_counts(cfg["experts"], cfg["m_lo"], cfg["m_hi"], cfg["seed"])
    G, N, K = cfg["experts"], cfg["N"], cfg["K"]
    print(f"\ndecode {G} experts, {int(off[-1])} rows, N {N}, K {K}", flush=True)
    outl = workloads.outlier_channels(K, cfg["seed"], cfg["outlier_frac"], cfg["outlier_count"])
    A = workloads.act_rows(np.arange(int(off[-1])), K, cfg["seed"], cfg["act_std"], outl,
                           cfg["outlier_mult"])
    f = fq()
    w = torch.empty((G, N, K), dtype=torch.bfloat16, device=DEV)
    for e in range(G):
        w[e] = workloads.expert_weight_torch(e, N, K, cfg["seed"], cfg["w_std"], DEV)
    aq, as_ = f.quantize_act(to_dev_bf16(A))
    wq, ws = f.quantize_weight(w.view(G * N, K))
    wq, ws = wq.view(G, N, K), ws.view(G, N // 128, K // 128)
    d_off = torch.from_numpy(off).to(DEV)
    c = f.grouped_gemm(aq, as_, d_off, wq, ws, out_dtype=torch.bfloat16)
    cp = f.grouped_gemm(aq, as_, d_off, wq, ws, out_dtype=torch.bfloat16, precise=True)
    torch.cuda.synchronize()
    ch, chp = _f64(c), _f64(cp)
    qa, sa = oquant.quantize_act(A)
    assert np.array_equal(host(aq), qa), "activation codes"
    assert np.array_equal(host(as_).view(np.uint32), sa.view(np.uint32)), "activation scales"
    within, total, worst, worst_fast = 0, 0, 0.0, 0.0
    for e in range(G):
        qw, sw = oquant.quantize_weight(bf16_to_bits(w[e]))
        assert np.array_equal(host(wq[e]), qw), f"expert {e} weight codes"
        assert np.array_equal(host(ws[e]).view(np.uint32), sw.view(np.uint32)), \
            f"expert {e} weight scales"
        r0, r1 = int(off[e]), int(off[e + 1])
        ref = ogemm.gemm(qa[r0:r1], sa[:, r0:r1], qw, sw)
        absb = ogemm.abs_bound(qa[r0:r1], sa[:, r0:r1], qw, sw)
        r = assert_gemm_strict(chp[r0:r1], qa[r0:r1], sa[:, r0:r1], qw, sw, out="bf16",
                               what=f"decode precise expert {e}, every output", ref=ref,
                               absb=absb)
        worst = max(worst, r["max_err_over_tol"])
        rf = assert_gemm_bounded(ch[r0:r1], qa[r0:r1], sa[:, r0:r1], qw, sw, out="bf16",
                                 what=f"decode fast path expert {e}, every output", ref=ref,
                                 absb=absb, native=True)
        worst_fast = max(worst_fast, rf["max_err_over_bound"])
        within += rf["strict_fraction"] * ref.size
        total += ref.size
    print(f"decode: {total} outputs; precise max err / tolerance {worst:.3g}; fast path max "
          f"err / its bound {worst_fast:.3g}, within 1e-5*sum|a||b|: {within / total:.6f}")


def _layer_backward_inputs():
    """The dense layer's backward operands: X and W of the dense workload
    (4096 tokens x 7168, 4096 x 7168) and an upstream gradient dY of 4096 x
    4096, N(0, 0.01^2) (seed 22, as the Wgrad test of test_gpu_backward)."""
    X, W = workloads.dense_inputs("dense")
    M, N = X.shape[0], W.shape[0]
    dY = workloads.bf16_bits(
        (np.random.default_rng(22).standard_normal((M, N)) * 1e-2).astype(np.float32))
    return X, W, dY


def test_dgrad_dense_layer_every_output():
    """dX = dY W (4096 x 7168, inner dimension 4096): fp8q_gemm and
    fp8q_gemm_precise on quantize_act(dY) and quantize_weight_t(W), every
    output, against the oracle composed the same way."""
    X, W, dY = _layer_backward_inputs()
    print(f"\ndgrad {dY.shape[0]}x{W.shape[1]}x{dY.shape[1]}", flush=True)
    f = fq()
    qd, sd = f.quantize_act(to_dev_bf16(dY))
    qwt, swt = f.quantize_weight_t(to_dev_bf16(W))
    dx = f.gemm(qd, sd, qwt, swt)
    dxp = f.gemm(qd, sd, qwt, swt, precise=True)
    torch.cuda.synchronize()
    od = oquant.quantize_act(dY)
    owt = oquant.quantize_weight_t(W)
    assert np.array_equal(host(qd), od[0]) and np.array_equal(host(sd).view(np.uint32),
                                                              od[1].view(np.uint32))
    assert np.array_equal(host(qwt), owt[0]) and np.array_equal(host(swt).view(np.uint32),
                                                                owt[1].view(np.uint32))
    ref = ogemm.gemm(*od, *owt)
    absb = ogemm.abs_bound(*od, *owt)
    rp = assert_gemm_strict(_f64(dxp), *od, *owt, what="dgrad precise, every output",
                            ref=ref, absb=absb)
    rf = assert_gemm_bounded(_f64(dx), *od, *owt, what="dgrad fast path, every output",
                             ref=ref, absb=absb, native=True)
    print(f"dgrad precise: {rp}; fast path: {rf}")


def test_wgrad_dense_layer_every_output():
    """dW = dY^T X (4096 x 7168, inner dimension the 4096 tokens):
    fp8q_gemm_rowscaled and fp8q_gemm_rowscaled_precise on quantize_act_t(dY)
    and quantize_act_t(X), every output, against the oracle composed the same
    way (row-group scales on both operands)."""
    X, W, dY = _layer_backward_inputs()
    print(f"\nwgrad {dY.shape[1]}x{X.shape[1]}x{dY.shape[0]}", flush=True)
    f = fq()
    qdt, sdt = f.quantize_act_t(to_dev_bf16(dY))
    qxt, sxt = f.quantize_act_t(to_dev_bf16(X))
    dw = f.gemm_rowscaled(qdt, sdt, qxt, sxt)
    dwp = f.gemm_rowscaled(qdt, sdt, qxt, sxt, precise=True)
    torch.cuda.synchronize()
    odt = oquant.quantize_act_t(dY)
    oxt = oquant.quantize_act_t(X)
    for (q, s), (oq, os_) in (((qdt, sdt), odt), ((qxt, sxt), oxt)):
        assert np.array_equal(host(q), oq) and np.array_equal(host(s).view(np.uint32),
                                                              os_.view(np.uint32))
    ref = ogemm.gemm_rowscaled(*odt, *oxt)
    absb = ogemm.abs_bound_rowscaled(*odt, *oxt)
    rp = assert_gemm_strict(_f64(dwp), *odt, *oxt, what="wgrad precise, every output",
                            rowscaled=True, ref=ref, absb=absb)
    rf = assert_gemm_bounded(_f64(dw), *odt, *oxt, what="wgrad fast path, every output",
                             rowscaled=True, ref=ref, absb=absb, native=True)
    print(f"wgrad precise: {rp}; fast path: {rf}")
