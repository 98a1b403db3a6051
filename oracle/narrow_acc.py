"""Emulator of a narrow fixed-point FP8 accumulator (accuracy study only).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity of the absolute
error magnitudes is UNPINNED: the pages print no error figure; only the
limits, hand cases and the trend below are pinned.

What is emulated ([whybe-72410], fixed-point accumulation passage;
[goodkr-2169793], limited accumulation bit-width passage): inside the matrix
unit the products are aligned to the largest exponent by a sign-fill right
shift and only the top W = 14 bits of each are kept, the rest truncated; the
error grows with K.  [pkd-78017] (increased-precision accumulation passage)
sets the promotion interval at 128 elements = four WGMMAs, so one aligned
step takes 32 products.

Readings (also in the design notes):
* the running accumulator takes part in each alignment step together with the
  32 new products (otherwise promotion every 128 could not help);
* "sign-fill right shift ... truncate" on a two's-complement value is floor;
* a step's unit is 2^(E - W + 1) with E = max floor(log2 |t|) over the
  step's non-zero terms.

Arithmetic is exact: every E4M3 value times 2^9 is an integer, so every
product is an integer in units of 2^-18, and sums stay far below 2^53.
"""

import numpy as np

from . import e4m3
from .quant import GROUP

UNIT_EXP = -18  # products are integers in units of 2^-18
K_STEP = 32     # products per aligned step (one FP8 WGMMA's K depth)


def int_values(q):
    """dec(q) * 2^9 as int64 (exact: every E4M3 value is a multiple of 2^-9)."""
    v = e4m3.decode(q) * 512.0
    iv = v.astype(np.int64)
    assert np.all(iv == v), "E4M3 values must be multiples of 2^-9"
    return iv


def _floor_log2(absval):
    """floor(log2 x) for positive integers held exactly in float64."""
    _, ex = np.frexp(absval.astype(np.float64))
    return ex - 1


def aligned_step(acc, terms, width):
    """One fixed-point step: align acc and the new terms to their largest
    exponent, keep the top ``width`` bits of each (floor), and add.

    acc: int64[P]; terms: int64[P][T]; width: int or None (None = exact).
    """
    T = np.concatenate([acc[:, None], terms], axis=1)
    if width is None:
        return T.sum(axis=1)
    mag = np.abs(T)
    nz = mag > 0
    e = np.where(nz, _floor_log2(np.where(nz, mag, 1)), np.iinfo(np.int64).min // 2)
    E = e.max(axis=1)
    shift = np.maximum(E - width + 1, 0)  # bits below the kept window
    unit = (np.int64(1) << shift)[:, None]
    kept = np.floor_divide(T, unit) * unit  # floor = sign-fill right shift
    return kept.sum(axis=1)


def narrow_chain(pa, pb, width, k_step=K_STEP, restart_every=None):
    """Run the aligned-step accumulation over all of K for P (row, row) pairs.

    pa, pb: int64[P][K] integer operand values (dec * 2^9).
    restart_every: None, or a K interval after which the chain result is
    handed out and the accumulator restarts at zero.
    Returns int64[P][n_out] chain results in units of 2^-18.
    """
    P, K = pa.shape
    outs = []
    acc = np.zeros(P, dtype=np.int64)
    for k0 in range(0, K, k_step):
        terms = pa[:, k0:k0 + k_step] * pb[:, k0:k0 + k_step]
        acc = aligned_step(acc, terms, width)
        if restart_every is not None and (k0 + k_step) % restart_every == 0:
            outs.append(acc)
            acc = np.zeros(P, dtype=np.int64)
    if restart_every is None or K % restart_every:
        outs.append(acc)
    return np.stack(outs, axis=1)


def promoted_dot(qa_rows, sa_rows, qw_rows, sw_rows, width, k_step=K_STEP):
    """Fine-grained quantization + narrow accumulation inside each 128-K chunk
    + FP32 promotion: acc32 += fl32(chunk * fl32(s_a * s_w)).

    qa_rows, qw_rows: uint8[P][K] (row of A and row of W for each output);
    sa_rows: float32[P][K/128]; sw_rows: float32[P][K/128].
    Returns float32[P].
    """
    pa = int_values(qa_rows)
    pb = int_values(qw_rows)
    chunks = narrow_chain(pa, pb, width, k_step, restart_every=GROUP)
    chunk_val = np.ldexp(chunks.astype(np.float64), UNIT_EXP).astype(np.float32)
    acc = np.zeros(pa.shape[0], dtype=np.float32)
    for g in range(chunks.shape[1]):
        sc = (sa_rows[:, g] * sw_rows[:, g]).astype(np.float32)
        term = (chunk_val[:, g] * sc).astype(np.float32)
        acc = (acc + term).astype(np.float32)
    return acc


def per_tensor_dot(qa_rows, sa, qw_rows, sw, width, k_step=K_STEP):
    """Per-tensor-scaled operands, one narrow chain over all of K, scales
    applied at the end: fl32(fl32(chain) * fl32(sa * sw)).  Returns float32[P]."""
    pa = int_values(qa_rows)
    pb = int_values(qw_rows)
    chain = narrow_chain(pa, pb, width, k_step, restart_every=None)[:, 0]
    val = np.ldexp(chain.astype(np.float64), UNIT_EXP).astype(np.float32)
    sc = np.float32(np.float32(sa) * np.float32(sw))
    return (val * sc).astype(np.float32)
