"""OCP E4M3 (a.k.a. E4M3FN) codec, written from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Format ([goodkr-2169793], mixed-precision framework passage: E4M3 -- a 4-bit
exponent and a 3-bit mantissa -- is used for every tensor): one sign bit S,
exponent field E (4 bits, bias 7), mantissa field M (3 bits).

* E == 0            : subnormal, value (-1)^S * (M / 8) * 2^(1 - 7) = (-1)^S * M * 2^-9
* 1 <= E <= 15      : normal,    value (-1)^S * (1 + M / 8) * 2^(E - 7)
* E == 15 and M == 7: NaN (S.1111.111); the format has no infinities.

So the largest finite magnitude is (1 + 6/8) * 2^8 = 448 (code 0x7E), the
smallest normal 2^-6 (0x08) and the smallest subnormal 2^-9 (0x01).

Encoding (the reading used throughout: round to nearest, ties to even, the
method's stated rounding): a finite real v maps to the finite E4M3 value
nearest to it; when two are equally near, the one whose code has a zero least
significant bit wins.  Magnitudes above 448 saturate to 448.  A result of zero
keeps the sign of v (so -tiny and -0.0 give 0x80).
"""

import numpy as np

NAN_CODES = (0x7F, 0xFF)


def _decode_code(b):
    """Value of one code byte, straight from the field definitions."""
    sign = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


#: float64[256]: value of every code byte (NaN at 0x7F and 0xFF).
DECODE_TABLE = np.array([_decode_code(b) for b in range(256)], dtype=np.float64)

#: the 127 non-negative finite values, codes 0x00..0x7E, strictly increasing.
_POS_VALUES = DECODE_TABLE[:0x7F].copy()

#: largest finite magnitude, read off the table (not typed in).
MAX_FINITE = float(_POS_VALUES[-1])


def decode(q):
    """E4M3 code bytes (any integer array) -> float64 values."""
    return DECODE_TABLE[np.asarray(q, dtype=np.uint8)]


def encode(v):
    """Round finite float values to E4M3 codes (RNE, saturating, signed zero).

    ``v`` may be float32 or float64; every float32 value is exact in float64
    and the candidate values and their midpoints (at most 5 significant bits)
    are exact in float64 too, so each comparison below is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("encode: non-finite input is outside the codec's contract")
    mag = np.abs(v)
    # hi = index of the first table value >= mag; lo = hi - 1.
    hi = np.searchsorted(_POS_VALUES, mag, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)  # saturate above 448
    lo = np.maximum(hi - 1, 0)
    t_lo = _POS_VALUES[lo]
    t_hi = _POS_VALUES[hi]
    mid = 0.5 * (t_lo + t_hi)
    pick_hi = mag > mid
    tie = mag == mid
    # On a tie take the candidate with the even code (hi and lo differ by one).
    pick_hi = pick_hi | (tie & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo)
    # Saturation: with hi clamped to the last index, a magnitude above 448
    # would still compare against the 416/448 midpoint; force it to 448.
    code = np.where(mag >= MAX_FINITE, len(_POS_VALUES) - 1, code)
    code = code.astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def nearest_bruteforce(v):
    """Slow reference: argmin over all 127 finite magnitudes (for tests).

    Exact for |v| >= 2^-12 (all differences fit in float64); anything smaller
    is nearer to 0 than to 2^-9 and returns the signed zero.
    """
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    d = np.abs(mag[:, None] - _POS_VALUES[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equal distances prefer an even code
    even = (np.arange(len(_POS_VALUES)) & 1) == 0
    cand_even = cand & even[None, :]
    use_even = cand_even.any(axis=1)
    idx_even = np.argmax(cand_even, axis=1)
    idx_any = np.argmax(cand, axis=1)
    code = np.where(use_even, idx_even, idx_any)
    code = np.where(mag < 2.0 ** -12, 0, code)
    code = np.where(mag >= MAX_FINITE, len(_POS_VALUES) - 1, code)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code.astype(np.uint8) | sign).astype(np.uint8)
