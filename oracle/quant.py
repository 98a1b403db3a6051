"""Fine-grained quantizers: 1x128 activation groups and 128x128 weight blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ([goodkr-2169793], fine-grained quantization passage): the
max-abs value is taken online for every 1x128 activation tile (one row, 128
consecutive K) and every 128x128 weight block (128 rows of N by 128 K); the
scaling factor is derived from it so that the max-abs maps onto the largest
FP8 value, and the group is cast to FP8 (E4M3).  The scale is kept per group
along the inner dimension K so the GEMM can dequantize on the general ALUs
([goodkr-2169793], limited accumulation bit-width passage).

Readings taken where the pages leave a step open (each is also listed in the
design notes):

* FP32-scale mode: ``inv = fl32(448 / amax)`` and ``s = fl32(amax / 448)``, both
  IEEE round-to-nearest-even single-precision divisions, and
  ``q = E4M3_RNE(fl32(x * inv))``.  "Scale the max-abs to the FP8 maximum" is
  read as a multiply by 448/amax; the stored dequantization scale is
  amax/448.  Decisions that pick an integer code are taken in FP32 on both
  sides.
* A group whose ``inv`` is not finite (amax == 0, or amax so small that 448/amax
  overflows FP32) is "flushed": ``s = 0`` and every code is a signed zero.
* Power-of-two mode ([whybe-72410], scaling factors that are integral powers of
  two): ``s = 2^e`` with e the smallest integer such that 448 * 2^e >= amax, and
  ``q = E4M3_RNE(x * 2^-e)`` (the scaling is exact).  amax == 0 gives s = 0.
* FP32 arithmetic keeps subnormals (no flush-to-zero); numpy float32 does.

Layouts (the C boundary's): activations x[M][K] -> q[M][K], s[K/128][M]
(group-major); weights w[N][K] -> q[N][K], s[N/128][K/128].
"""

import numpy as np

from . import e4m3

GROUP = 128  # 1x128 activation tiles, 128x128 weight blocks
FP8_MAX = np.float32(e4m3.MAX_FINITE)  # 448, from the codec's table


def bf16_bits_to_f32(bits):
    """BF16 bit patterns (uint16) -> float32 values (exact widening)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _flushed_codes(x):
    """Signed zero codes for a flushed group: 0x00 or 0x80 by the sign of x."""
    return (np.signbit(x).astype(np.uint8) << 7).astype(np.uint8)


def _scale_group_f32(x, amax):
    """FP32-scale rule for values ``x`` (float32) whose groups have max-abs
    ``amax`` (float32, broadcast against x).  Returns (codes, s)."""
    with np.errstate(divide="ignore", over="ignore"):
        inv = FP8_MAX / amax  # float32 / float32: IEEE RNE
    flushed = ~np.isfinite(inv)
    s = np.where(flushed, np.float32(0.0), amax / FP8_MAX).astype(np.float32)
    inv_safe = np.where(flushed, np.float32(0.0), inv).astype(np.float32)
    y = (x * inv_safe).astype(np.float32)  # float32 * float32: IEEE RNE
    codes = e4m3.encode(y)
    codes = np.where(flushed, _flushed_codes(x), codes).astype(np.uint8)
    return codes, s


def pow2_exponent(amax):
    """Smallest integer e with 448 * 2^e >= amax, for amax > 0 (float array).

    Write amax = f * 2^E exactly with f in [1, 2).  448 = 1.75 * 2^8, so
    e = E - 8 when f <= 1.75 and e = E - 7 otherwise.
    """
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(amax)  # amax = m * 2^ex, m in [0.5, 1)
    f = 2.0 * m
    E = ex - 1
    return np.where(f <= 1.75, E - 8, E - 7).astype(np.int64)


def _scale_group_pow2(x, amax):
    """Power-of-two rule.  Returns (codes, s)."""
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax)
    e = pow2_exponent(safe)
    s = np.where(zero, 0.0, np.ldexp(1.0, e)).astype(np.float32)
    y = np.ldexp(x.astype(np.float64), -e)  # exact
    codes = e4m3.encode(y)
    codes = np.where(zero, _flushed_codes(x), codes).astype(np.uint8)
    return codes, s


def quantize_act(x_bits, mode="f32"):
    """1x128 activation quantization.

    x_bits: uint16[M][K] BF16 bit patterns, K % 128 == 0.
    Returns q: uint8[M][K] E4M3 codes, s: float32[K/128][M].
    """
    x = bf16_bits_to_f32(x_bits)
    M, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    G = K // GROUP
    xg = x.reshape(M, G, GROUP)
    if mode not in ("f32", "pow2"):
        raise ValueError(mode)
    amax = np.abs(xg).max(axis=2, keepdims=True) if M else np.zeros((0, G, 1), np.float32)
    rule = _scale_group_f32 if mode == "f32" else _scale_group_pow2
    codes, s = rule(xg, amax)
    q = codes.reshape(M, K)
    s = np.broadcast_to(s, (M, G, 1))[:, :, 0].T.copy()  # [G][M]
    return q, s.astype(np.float32)


def quantize_weight(w_bits, mode="f32"):
    """128x128 weight-block quantization.

    w_bits: uint16[N][K] BF16 bit patterns, N % 128 == 0, K % 128 == 0.
    Returns q: uint8[N][K] E4M3 codes, s: float32[N/128][K/128].
    """
    w = bf16_bits_to_f32(w_bits)
    N, K = w.shape
    if N % GROUP or K % GROUP:
        raise ValueError("N and K must be multiples of 128")
    NB, KB = N // GROUP, K // GROUP
    wb = w.reshape(NB, GROUP, KB, GROUP)
    amax = np.abs(wb).max(axis=(1, 3), keepdims=True) if N else np.zeros((0, 1, KB, 1), np.float32)
    if mode not in ("f32", "pow2"):
        raise ValueError(mode)
    rule = _scale_group_f32 if mode == "f32" else _scale_group_pow2
    codes, s = rule(wb, amax)
    q = codes.reshape(N, K)
    s = np.broadcast_to(s, (NB, 1, KB, 1))[:, 0, :, 0].copy()
    return q, s.astype(np.float32)


def quantize_act_t(x_bits, mode="f32"):
    """Transposed activation quantization for the weight-gradient GEMM, whose
    inner dimension is the token dimension M ([goodkr-2169793], mixed-precision
    framework passage: Fprop, Dgrad and Wgrad all run in FP8; the scales are
    per group along each GEMM's inner dimension).  Groups are 128 consecutive
    rows of one column: the 1x128 rule applied to x^T.

    x_bits: uint16[M][K], M % 128 == 0.
    Returns q_t: uint8[K][M] (codes of x^T), s_t: float32[M/128][K].
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.shape[0] % GROUP:
        raise ValueError("M must be a multiple of 128")
    return quantize_act(np.ascontiguousarray(x_bits.T), mode)


def quantize_weight_t(w_bits, mode="f32"):
    """Transposed weight quantization for the activation-gradient GEMM
    (dX = dY W uses W^T as its weight operand): the 128x128 block rule applied
    to w^T, i.e. the same blocks with their codes transposed.

    w_bits: uint16[N][K].  Returns q_t: uint8[K][N], s_t: float32[K/128][N/128].
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    return quantize_weight(np.ascontiguousarray(w_bits.T), mode)


def dequantize_act(q, s):
    """dec(q) * s as float64[M][K] (s laid out [K/128][M])."""
    v = e4m3.decode(q)
    M, K = v.shape
    return v * np.repeat(s.T.astype(np.float64), GROUP, axis=1)


def dequantize_weight(q, s):
    """dec(q) * s as float64[N][K] (s laid out [N/128][K/128])."""
    v = e4m3.decode(q)
    full = np.repeat(np.repeat(s.astype(np.float64), GROUP, axis=0), GROUP, axis=1)
    return v * full


def quantize_tensor(x_bits):
    """Per-tensor quantization (the prior art the fine-grained scheme replaces,
    [goodkr-2169793] fine-grained quantization passage): one FP32-mode scale
    from the max-abs of the whole tensor.  Returns (q uint8[...], s float32)."""
    x = bf16_bits_to_f32(x_bits)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    codes, s = _scale_group_f32(x, amax)
    return codes, np.float32(s)
