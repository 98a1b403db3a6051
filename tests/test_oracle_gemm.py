"""Pins for the oracle's block-scaled GEMM and grouped GEMM (CPU only).

Pinned against: exact rational arithmetic (Fractions) on tiny shapes, an
independent int64 evaluation of every chunk partial, the K = 128 special case,
a torch float64 matmul when all scales are 1, linearity in one scale, and the
flushed-group rule.
"""

from fractions import Fraction

import numpy as np
import torch

import workloads
from oracle import e4m3, gemm, quant


def _quantized(M, N, K, seed, mode="f32"):
    rng = np.random.default_rng(seed)
    A = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = workloads.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    qa, sa = quant.quantize_act(A, mode)
    qw, sw = quant.quantize_weight(W, mode)
    return qa, sa, qw, sw


def test_exact_rational_bruteforce():
    qa, sa, qw, sw = _quantized(6, 128, 384, 1)
    C = gemm.gemm(qa, sa, qw, sw)
    bound = gemm.abs_bound(qa, sa, qw, sw)
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.DECODE_TABLE]
    for m in range(6):
        for n in (0, 1, 77, 127):
            exact = Fraction(0)
            for k in range(384):
                g = k // 128
                exact += (Fraction(float(sa[g, m])) * Fraction(float(sw[n // 128, g]))
                          * dec[qa[m, k]] * dec[qw[n, k]])
            # one float64 rounding per chunk add: at most 3 * 2^-53 of the bound
            assert abs(Fraction(float(C[m, n])) - exact) <= Fraction(float(bound[m, n])) * Fraction(4, 2**53)


def test_chunk_partials_exact_against_int64():
    qa, sa, qw, sw = _quantized(33, 256, 512, 2)
    ia = (e4m3.decode(qa) * 512).astype(np.int64)
    iw = (e4m3.decode(qw) * 512).astype(np.int64)
    for g, P in gemm.chunk_partials(qa, qw):
        ks = slice(g * 128, (g + 1) * 128)
        Pi = ia[:, ks] @ iw[:, ks].T  # integer, units of 2^-18
        assert np.array_equal(P, np.ldexp(Pi.astype(np.float64), -18))
        assert np.all(np.abs(Pi) < 2**53)


def test_k128_reduces_to_scaled_product():
    qa, sa, qw, sw = _quantized(17, 256, 128, 3)
    C = gemm.gemm(qa, sa, qw, sw)
    A = e4m3.decode(qa)
    W = e4m3.decode(qw)
    ref = sa[0].astype(np.float64)[:, None] * np.repeat(sw[:, 0].astype(np.float64), 128)[None, :] * (A @ W.T)
    assert np.array_equal(C, ref)


def test_unit_scales_match_torch_matmul():
    qa, _, qw, _ = _quantized(40, 128, 640, 4)
    sa = np.ones((5, 40), np.float32)
    sw = np.ones((1, 5), np.float32)
    C = gemm.gemm(qa, sa, qw, sw)
    ref = (torch.from_numpy(qa).view(torch.float8_e4m3fn).to(torch.float64)
           @ torch.from_numpy(qw).view(torch.float8_e4m3fn).to(torch.float64).T).numpy()
    assert np.array_equal(C, ref)


def test_linear_in_one_group_scale_and_flushed_group():
    qa, sa, qw, sw = _quantized(8, 128, 512, 5)
    C = gemm.gemm(qa, sa, qw, sw)
    A = e4m3.decode(qa)
    W = e4m3.decode(qw)
    g, m = 2, 3
    contrib = float(sa[g, m]) * float(sw[0, g]) * (A[m, 256:384] @ W[:, 256:384].T)
    sa2 = sa.copy()
    sa2[g, m] *= 2
    C2 = gemm.gemm(qa, sa2, qw, sw)
    assert np.allclose(C2[m] - C[m], contrib, rtol=0, atol=1e-12 * np.abs(C[m]).max())
    others = np.arange(8) != m
    assert np.array_equal(C2[others], C[others])
    # a flushed activation group (codes zero, scale zero) contributes nothing
    qa3, sa3 = qa.copy(), sa.copy()
    qa3[m, 256:384] = 0
    sa3[g, m] = 0
    C3 = gemm.gemm(qa3, sa3, qw, sw)
    assert np.allclose(C3[m], C[m] - contrib, rtol=0, atol=1e-12 * np.abs(C[m]).max())


def test_sign_and_transpose_sensitivity():
    """Swapping operand roles transposes the output; negating A negates C."""
    qa, sa, qw, sw = _quantized(128, 128, 256, 6)
    C = gemm.gemm(qa, sa, qw, sw)
    # W's block scales, spread over its 128 rows, serve as activation scales
    sa_blk = np.repeat(sw[0][:, None], 128, axis=1)  # [K/128][M=128]
    Ct = gemm.gemm(qw, sa_blk, qa, np.ones((1, 2), np.float32))
    Cr = gemm.gemm(qa, np.ones_like(sa), qw, sw)
    assert np.array_equal(Ct.T, Cr)
    Cn = gemm.gemm(qa ^ np.uint8(0x80), sa, qw, sw)
    assert np.array_equal(Cn, -C)


def test_grouped_equals_per_expert_dense():
    rng = np.random.default_rng(8)
    G, N, K = 5, 128, 256
    counts = np.array([3, 0, 17, 1, 0])
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    Mt = int(off[-1]) + 4  # rows past off[G] are not part of the result
    A = workloads.bf16_bits(rng.standard_normal((Mt, K)).astype(np.float32))
    qa, sa = quant.quantize_act(A)
    qws, sws = [], []
    for e in range(G):
        W = workloads.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        q, s = quant.quantize_weight(W)
        qws.append(q)
        sws.append(s)
    qw, sw = np.stack(qws), np.stack(sws)
    C = gemm.grouped_gemm(qa, sa, off, qw, sw)
    for e in range(G):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            assert np.array_equal(C[r0:r1], gemm.gemm(qa[r0:r1], sa[:, r0:r1], qw[e], sw[e]))
    assert np.all(np.isnan(C[off[-1]:]))


def test_bf16_rounding_helpers():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -3.0 - 2.0 ** -7, 1e-3])
    r = gemm.round_to_bf16(v)
    assert r[0] == 1.0
    assert r[1] == 1.0  # tie -> even
    assert r[2] == 1.0 + 2 * 2.0 ** -7  # tie -> even (up)
    assert r[3] == -3.0  # -3 - 2^-7: half ulp at 2 is 2^-7 -> tie -> even (-3.0)
    ref = torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(r, ref)
    assert gemm.bf16_half_ulp(np.array([1.0]))[0] == 2.0 ** -8


def test_bf16_reference_exact_rational_bruteforce():
    """gemm_bf16 against exact rational sums of the BF16 values (tiny shape,
    signed values, an x50 outlier column)."""
    rng = np.random.default_rng(41)
    M, N, K = 5, 7, 256
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, 3] *= 50
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = workloads.bf16_bits(a)
    W = workloads.bf16_bits(w)
    C = gemm.gemm_bf16(A, W)
    bound = gemm.abs_bound_bf16(A, W)
    av = quant.bf16_bits_to_f32(A)
    wv = quant.bf16_bits_to_f32(W)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(av[m, k])) * Fraction(float(wv[n, k])) for k in range(K))
            assert abs(Fraction(float(C[m, n])) - exact) <= Fraction(float(bound[m, n])) * Fraction(K, 2**53)
            # the bound itself is the sum of magnitudes
            mag = sum(abs(Fraction(float(av[m, k])) * Fraction(float(wv[n, k]))) for k in range(K))
            assert abs(Fraction(float(bound[m, n])) - mag) <= mag * Fraction(K, 2**53)


def test_bf16_reference_permutation_picks_columns():
    """W = a permutation matrix P (w[n][k] = 1 iff k = p[n]): C[m][n] = a[m][p[n]].
    A transposed operand or a swapped index would pick the wrong entries."""
    rng = np.random.default_rng(42)
    M, K = 9, 384
    N = 128
    a = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    p = rng.permutation(K)[:N]
    w = np.zeros((N, K), dtype=np.float32)
    w[np.arange(N), p] = 1.0
    C = gemm.gemm_bf16(a, workloads.bf16_bits(w))
    assert np.array_equal(C, quant.bf16_bits_to_f32(a)[:, p].astype(np.float64))


def test_rowscaled_gemm_exact_and_reduces_to_block_scaled():
    """gemm_rowscaled: exact rational brute force on a tiny case, and equal to
    gemm() when the second operand's row scales are constant over 128-row
    blocks (sb[g][n] = sw[n // 128][g])."""
    rng = np.random.default_rng(12)
    M, N, K = 4, 256, 384
    A = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    B = workloads.bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    qa, sa = quant.quantize_act(A)
    qb, sb = quant.quantize_act(B)     # row-group scales [K/128][N]
    C = gemm.gemm_rowscaled(qa, sa, qb, sb)
    bound = gemm.abs_bound_rowscaled(qa, sa, qb, sb)
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.DECODE_TABLE]
    for m in range(M):
        for n in (0, 3, 129, 255):
            exact = sum(Fraction(float(sa[k // 128, m])) * Fraction(float(sb[k // 128, n]))
                        * dec[qa[m, k]] * dec[qb[n, k]] for k in range(K))
            assert abs(Fraction(float(C[m, n])) - exact) <= Fraction(float(bound[m, n])) * Fraction(4, 2**53)
    qw, sw = quant.quantize_weight(workloads.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32)))
    sb_blocks = np.repeat(sw, 128, axis=0).T.copy()  # [K/128][N]
    assert np.array_equal(gemm.gemm_rowscaled(qa, sa, qw, sb_blocks), gemm.gemm(qa, sa, qw, sw))


def test_backward_gemms_of_a_linear_layer():
    """Dgrad and Wgrad of Y = X W^T through the quantized operands agree with
    the float64 gradients to within the FP8 quantization error: a check that
    the operands and their transposes are wired the right way round."""
    rng = np.random.default_rng(13)
    M, N, K = 256, 256, 384
    X = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = workloads.bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    dY = workloads.bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    Xf, Wf, dYf = (quant.bf16_bits_to_f32(t).astype(np.float64) for t in (X, W, dY))
    # Dgrad: dX = dY W  (inner dimension N)
    qd, sd = quant.quantize_act(dY)
    qwt, swt = quant.quantize_weight_t(W)
    dX = gemm.gemm(qd, sd, qwt, swt)
    ref = dYf @ Wf
    assert np.linalg.norm(dX - ref) / np.linalg.norm(ref) < 0.06
    # Wgrad: dW = dY^T X  (inner dimension M, both operands grouped along M)
    qa, sa = quant.quantize_act_t(dY)   # dY^T [N][M]
    qb, sb = quant.quantize_act_t(X)    # X^T  [K][M]
    dW = gemm.gemm_rowscaled(qa, sa, qb, sb)
    refw = dYf.T @ Xf
    assert np.linalg.norm(dW - refw) / np.linalg.norm(refw) < 0.06
    # a transposed operand would be far off
    assert np.linalg.norm(dW.T[:N, :N] - refw[:N, :N]) / np.linalg.norm(refw[:N, :N]) > 0.5


def test_abs_bound_exact_rational_bruteforce():
    """abs_bound (the tolerance's sum_k |dec(a_k) s_a| |dec(w_k) s_w|) against a
    Fraction triple loop over the DECODED values: signed codes (the bound must
    take magnitudes), a flushed group (scale 0), subnormal codes, a negative
    scale (magnitude taken), and two weight blocks with different scales (a
    transposed or misindexed scale table fails)."""
    rng = np.random.default_rng(12)
    M, N, K = 5, 256, 384
    qa = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    qw = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x01      # no NaN codes; 0x01 is the smallest subnormal
    qw[(qw & 0x7F) == 0x7F] = 0x81
    sa = rng.uniform(0.5, 2.0, size=(K // 128, M)).astype(np.float32)
    sw = rng.uniform(0.5, 2.0, size=(N // 128, K // 128)).astype(np.float32)
    sa[1, 2] = 0.0                        # a flushed group
    sw[1, 0] = -sw[1, 0]                  # a sign the bound must drop
    got = gemm.abs_bound(qa, sa, qw, sw)
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.DECODE_TABLE]
    for m in range(M):
        for n in (0, 5, 127, 128, 200, 255):
            want = Fraction(0)
            for k in range(K):
                g = k // 128
                want += (abs(dec[qa[m, k]] * Fraction(float(sa[g, m])))
                         * abs(dec[qw[n, k]] * Fraction(float(sw[n // 128, g]))))
            # float64 accumulation over 3 chunks: within 4 * 2^-53 relative
            assert abs(Fraction(float(got[m, n])) - want) <= want * Fraction(4, 2**53), (m, n)
    assert np.all(got >= np.abs(gemm.gemm(qa, sa, qw, sw)))


def test_abs_bound_rowscaled_exact_rational_bruteforce():
    rng = np.random.default_rng(13)
    M, N, K = 4, 128, 256
    qa = rng.integers(0, 127, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    qb = rng.integers(0, 127, size=(N, K)).astype(np.uint8)
    sa = rng.uniform(0.5, 2.0, size=(K // 128, M)).astype(np.float32)
    sb = rng.uniform(0.5, 2.0, size=(K // 128, N)).astype(np.float32)
    got = gemm.abs_bound_rowscaled(qa, sa, qb, sb)
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.DECODE_TABLE]
    for m in range(M):
        for n in (0, 3, 64, 127):
            want = sum(abs(dec[qa[m, k]] * Fraction(float(sa[k // 128, m])))
                       * abs(dec[qb[n, k]] * Fraction(float(sb[k // 128, n]))) for k in range(K))
            assert abs(Fraction(float(got[m, n])) - want) <= want * Fraction(4, 2**53), (m, n)
