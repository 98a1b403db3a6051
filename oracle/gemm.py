"""Block-scaled FP8 GEMM with promotion every 128 K, evaluated exactly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed.  The operands are E4M3 codes with one scale per 1x128
activation group (s_a[g][m]) and one per 128x128 weight block
(s_w[n/128][g]).  For every 128-wide K interval g the FP8 products are summed
into a partial result P_g, which is then multiplied by the two scaling factors
and added into the FP32 accumulator ([whybe-57820], promotion passage;
[pkd-78017], 128 elements as the promotion interval; [goodkr-2169793],
per-group scaling along K dequantized on the general ALUs):

    C[m][n] = sum_g (s_a[g][m] * s_w[n // 128][g]) * P_g[m][n]
    P_g[m][n] = sum_{k in [128g, 128g + 128)} dec(qa[m][k]) * dec(qw[n][k])

This oracle evaluates that definition in float64.  Every E4M3 value is an
integer multiple of 2^-9 with at most 4 significant bits, so every product is
an integer multiple of 2^-18 below 2^18, and a sum of 128 of them needs fewer
than 53 bits: P_g is exact in float64 whatever the summation order (so a
library matmul may form it).  The scale product s_a * s_w (two FP32 values) is
exact in float64; the cross-chunk sum rounds once per chunk at 2^-53.
"""

import numpy as np

from . import e4m3
from .quant import GROUP


def chunk_partials(qa, qw):
    """Yield (g, P_g) for each 128-wide K chunk, P_g float64[M][N] (exact)."""
    A = e4m3.decode(qa)
    W = e4m3.decode(qw)
    K = A.shape[1]
    for g in range(K // GROUP):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        yield g, A[:, ks] @ W[:, ks].T


def gemm(qa, sa, qw, sw):
    """C (float64[M][N]) = sum over chunks of (s_a * s_w) * P_g.

    qa: uint8[M][K], sa: float32[K/128][M], qw: uint8[N][K], sw: float32[N/128][K/128].
    """
    M, K = qa.shape
    N = qw.shape[0]
    C = np.zeros((M, N), dtype=np.float64)
    for g, P in chunk_partials(qa, qw):
        row_scale = sa[g].astype(np.float64)[:, None]  # [M][1]
        col_scale = np.repeat(sw[:, g].astype(np.float64), GROUP)[None, :]  # [1][N]
        C += (row_scale * col_scale) * P
    return C


def abs_bound(qa, sa, qw, sw):
    """sum_k |dec(qa) s_a| * |dec(qw) s_w| per output (float64[M][N]).

    The acceptance test scales this by 1e-5: |C_gpu - C| <= 1e-5 * abs_bound.
    """
    qa_abs = qa & np.uint8(0x7F)
    qw_abs = qw & np.uint8(0x7F)
    return gemm(qa_abs, np.abs(sa), qw_abs, np.abs(sw))


def grouped_gemm(qa, sa, offsets, qw, sw):
    """Rows [offsets[e], offsets[e+1]) of qa use expert e's weights.

    qa: uint8[M_total][K]; sa: float32[K/128][M_total]; offsets: int[G+1];
    qw: uint8[G][N][K]; sw: float32[G][N/128][K/128].
    Rows at or past offsets[G] are not part of the result (returned as NaN).
    """
    M_total = qa.shape[0]
    N = qw.shape[1]
    C = np.full((M_total, N), np.nan, dtype=np.float64)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            C[r0:r1] = gemm(qa[r0:r1], sa[:, r0:r1], qw[e], sw[e])
    return C


def gemm_rowscaled(qa, sa, qb, sb):
    """Block-scaled GEMM whose both operands carry 1x128 row-group scales (the
    weight-gradient GEMM, dW = dY^T X: operands dY^T and X^T grouped along the
    tokens; [goodkr-2169793], mixed-precision framework passage):

        C[m][n] = sum_g (sa[g][m] * sb[g][n]) * P_g[m][n]

    qa: uint8[M][K], sa: float32[K/128][M], qb: uint8[N][K], sb: float32[K/128][N].
    """
    M, K = qa.shape
    N = qb.shape[0]
    C = np.zeros((M, N), dtype=np.float64)
    for g, P in chunk_partials(qa, qb):
        C += (sa[g].astype(np.float64)[:, None] * sb[g].astype(np.float64)[None, :]) * P
    return C


def abs_bound_rowscaled(qa, sa, qb, sb):
    """sum_k |dec(qa) s_a| * |dec(qb) s_b| per output (float64[M][N])."""
    return gemm_rowscaled(qa & np.uint8(0x7F), np.abs(sa), qb & np.uint8(0x7F), np.abs(sb))


def gemm_bf16(a_bits, w_bits):
    """BF16 reference GEMM: C (float64[M][N]) = sum_k a[m][k] * w[n][k].

    a_bits: uint16[M][K], w_bits: uint16[N][K] BF16 bit patterns.  This is the
    unquantized product the FP8 path is measured against ([goodkr-2169793],
    mixed-precision framework passage: FP8 GEMMs in place of BF16 ones).  A
    BF16 value has 8 significant bits, so every product is exact in float64;
    the sum over K rounds at 2^-53 relative to the running sum.
    """
    from .quant import bf16_bits_to_f32
    a = bf16_bits_to_f32(a_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    return a @ w.T


def abs_bound_bf16(a_bits, w_bits):
    """sum_k |a[m][k]| * |w[n][k]| (float64[M][N]), for the 1e-5 tolerance."""
    return gemm_bf16(np.asarray(a_bits, np.uint16) & np.uint16(0x7FFF),
                     np.asarray(w_bits, np.uint16) & np.uint16(0x7FFF))


def round_to_f32(c):
    """RNE of float64 values to float32 (numpy's cast is RNE)."""
    return np.asarray(c, dtype=np.float64).astype(np.float32)


def round_to_bf16(c):
    """RNE of float64 values straight to BF16 (8 significant bits), as float64.

    Normal range only (the GEMM outputs here are far from BF16's subnormals).
    """
    c = np.asarray(c, dtype=np.float64)
    m, ex = np.frexp(c)  # c = m * 2^ex, |m| in [0.5, 1)
    r = np.rint(m * 256.0)  # 8 significant bits, ties to even
    return np.ldexp(r, ex - 8)


def bf16_half_ulp(c):
    """Half a BF16 unit in the last place of |c| (float64)."""
    c = np.abs(np.asarray(c, dtype=np.float64))
    _, ex = np.frexp(np.where(c == 0, 1.0, c))
    return np.where(c == 0, 0.0, np.ldexp(1.0, ex - 9))
