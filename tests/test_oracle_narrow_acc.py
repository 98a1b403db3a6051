"""Pins for the narrow fixed-point accumulator emulator (CPU only).

The absolute error magnitudes are parity UNPINNED (the pages print none); what
is pinned: hand cases (tests/golden/narrow_acc_hand_cases.txt), the exact
limit (no truncation reproduces the exact GEMM's chunk sums), and the trend
that the pages state: the error of one long narrow chain grows with K while
promotion every 128 keeps it flat.
"""

import os

import numpy as np

import workloads
from oracle import gemm, narrow_acc, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "narrow_acc_hand_cases.txt")


def test_hand_cases():
    n = 0
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        w, acc, prod, expect = (int(t) for t in line.split())
        got = narrow_acc.aligned_step(np.array([acc], np.int64),
                                      np.full((1, 32), prod, np.int64), w)
        assert got[0] == expect, line
        n += 1
    assert n >= 4


def test_floor_not_round_to_zero():
    # -1 unit below the window floors to -unit, +1 floors to 0
    acc = np.array([1 << 20], np.int64)
    t = np.array([[1, -1]], np.int64)
    assert narrow_acc.aligned_step(acc, t, 14)[0] == (1 << 20) - (1 << 7)


def _rows(P, K, seed):
    rng = np.random.default_rng(seed)
    A = workloads.bf16_bits(rng.standard_normal((P, K)).astype(np.float32))
    W = workloads.bf16_bits(rng.standard_normal((P, K)).astype(np.float32))
    return A, W


def test_exact_width_reproduces_exact_chunks():
    A, W = _rows(16, 512, 1)
    qa, sa = quant.quantize_act(A)
    # weights as 1x128 groups per row too (each row its own "block" for this check)
    qw, sw = quant.quantize_act(W)
    pa = narrow_acc.int_values(qa)
    pb = narrow_acc.int_values(qw)
    chunks = narrow_acc.narrow_chain(pa, pb, None, restart_every=128)
    for g in range(4):
        ks = slice(g * 128, (g + 1) * 128)
        P = np.einsum("ik,ik->i", pa[:, ks], pb[:, ks])
        assert np.array_equal(chunks[:, g], P)
    # and the diagonal of the exact GEMM's chunk partials
    for g, Pg in gemm.chunk_partials(qa, qw):
        assert np.array_equal(np.ldexp(chunks[:, g].astype(np.float64), -18), np.diag(Pg))


def test_error_grows_with_k_without_promotion():
    """Per-tensor operands, one 14-bit chain over all of K (no promotion) versus
    1x128 groups with promotion every 128: relative to sum |a||b| the first
    error grows with K, the second stays small (the limited accumulation
    bit-width passage)."""
    errs_chain, errs_prom = [], []
    for K in (512, 4096, 16384):
        A, W = _rows(48, K, 100 + K)
        qt_a, st_a = quant.quantize_tensor(A)
        qt_w, st_w = quant.quantize_tensor(W)
        exact_t = narrow_acc.per_tensor_dot(qt_a, st_a, qt_w, st_w, None).astype(np.float64)
        narrow_t = narrow_acc.per_tensor_dot(qt_a, st_a, qt_w, st_w, 14).astype(np.float64)
        xa = quant.bf16_bits_to_f32(A).astype(np.float64)
        xw = quant.bf16_bits_to_f32(W).astype(np.float64)
        absum = np.einsum("ik,ik->i", np.abs(xa), np.abs(xw))
        errs_chain.append(np.median(np.abs(narrow_t - exact_t) / absum))
        qa, sa = quant.quantize_act(A)
        qw, sw = quant.quantize_act(W)
        prom = narrow_acc.promoted_dot(qa, sa.T, qw, sw.T, 14).astype(np.float64)
        exact_p = narrow_acc.promoted_dot(qa, sa.T, qw, sw.T, None).astype(np.float64)
        errs_prom.append(np.median(np.abs(prom - exact_p) / absum))
    assert errs_chain[0] < errs_chain[1] < errs_chain[2]
    assert errs_chain[2] > 4 * errs_chain[0]
    assert max(errs_prom) < errs_chain[2] / 8
