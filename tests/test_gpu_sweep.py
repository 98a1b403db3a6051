"""A seeded sweep of random shapes through every forward GEMM entry point, on
the GPU, against the oracle and against each other:

- fp8q_gemm within its a-priori bound (on one weight block of columns, the
  bound costing M*N*K work), fp8q_gemm_precise within 1e-5 * sum|a||b| on
  every output (both against the exact oracle);
- fp8q_gemm_fused equal to quantize-then-fp8q_gemm bit for bit;
- with power-of-two scales, fp8q_gemm_mfma_scaled equal to fp8q_gemm bit for
  bit;
- fp8q_grouped_gemm / _precise over random expert splits of the rows (empty
  experts included) equal, row by row, to the dense calls on each expert's
  rows and weights, bit for bit (every output's arithmetic is independent of
  the tiling).
Shapes: M in 1..320, N a multiple of 128 up to 512, K a multiple of 128 up
to 1280; scale mode and output type vary with the case.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import DEV, assert_gemm_bounded, assert_gemm_strict, fq, to_dev_bf16
from oracle import quant as oquant

pytestmark = pytest.mark.gpu

CASES = 12


def _case(i):
    rng = np.random.default_rng(90000 + i)
    M = int(rng.integers(1, 321))
    N = 128 * int(rng.integers(1, 5))
    K = 128 * int(rng.integers(1, 11))
    mode = "pow2" if i % 2 else "f32"
    out = "bf16" if i % 3 == 2 else "f32"
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(rng.choice([1.0, 30.0]))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return rng, M, N, K, mode, out, workloads.bf16_bits(a), workloads.bf16_bits(w)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _host64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape(i):
    rng, M, N, K, mode, out, A, W = _case(i)
    print(f"\ncase {i}: M={M} N={N} K={K} {mode} {out}", flush=True)
    f = fq()
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    a, w = to_dev_bf16(A), to_dev_bf16(W)
    aq, as_ = f.quantize_act(a, mode)
    wq, ws = f.quantize_weight(w, mode)
    c = f.gemm(aq, as_, wq, ws, out_dtype=dt)
    cp = f.gemm(aq, as_, wq, ws, out_dtype=dt, precise=True)
    cf = f.gemm_fused(a, wq, ws, mode, out_dtype=dt)
    cm = f.gemm(aq, as_, wq, ws, out_dtype=dt, mfma_scaled=True) if mode == "pow2" else None

    # grouped: the rows split over G experts (some empty), expert e's weights
    # are W with its rows rolled by e blocks, so experts differ
    G = int(rng.integers(1, 6))
    cuts = np.sort(rng.integers(0, M + 1, size=G - 1))
    off_h = np.concatenate([[0], cuts, [M]]).astype(np.int32)
    wq3 = torch.stack([torch.roll(wq, 128 * e, 0) for e in range(G)])
    ws3 = torch.stack([torch.roll(ws, e, 0) for e in range(G)])
    off = torch.from_numpy(off_h).to(DEV)
    cg = f.grouped_gemm(aq, as_, off, wq3, ws3, out_dtype=dt)
    cgp = f.grouped_gemm(aq, as_, off, wq3, ws3, out_dtype=dt, precise=True)
    torch.cuda.synchronize()

    assert torch.equal(_bits(cf), _bits(c)), "fused GEMM differs from quantize-then-GEMM"
    if cm is not None:
        assert torch.equal(_bits(cm), _bits(c)), "matrix-core-scaled GEMM differs from fp8q_gemm"
    for e in range(G):
        lo, hi = int(off_h[e]), int(off_h[e + 1])
        if hi == lo:
            continue
        ce = f.gemm(aq[lo:hi].contiguous(), as_[:, lo:hi].contiguous(), wq3[e], ws3[e], out_dtype=dt)
        cep = f.gemm(aq[lo:hi].contiguous(), as_[:, lo:hi].contiguous(), wq3[e], ws3[e],
                     out_dtype=dt, precise=True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(cg[lo:hi]), _bits(ce)), f"grouped expert {e} differs from dense"
        assert torch.equal(_bits(cgp[lo:hi]), _bits(cep)), f"precise grouped expert {e} differs"

    qa, sa = oquant.quantize_act(A, mode)
    qw, sw = oquant.quantize_weight(W, mode)
    assert np.array_equal(aq.cpu().numpy(), qa) and np.array_equal(wq.cpu().numpy(), qw)
    b = int(rng.integers(0, N // 128))
    cols = np.arange(128 * b, 128 * b + 128)
    r = assert_gemm_bounded(_host64(c), qa, sa, qw, sw, out=out, bound_cols=cols,
                            what=f"case {i} fast")
    rp = assert_gemm_strict(_host64(cp), qa, sa, qw, sw, out=out, what=f"case {i} precise")
    print(f"case {i}: fast {r}; precise {rp}")
