"""Pins for the oracle's 1x128 / 128x128 quantizers (CPU only).

Pinned against: the max-abs-to-448 invariant, the flushed-group rule, the
dequantization error bound, a PyTorch float32 + float8_e4m3fn pipeline
(independent library arithmetic), exact rational checks, brute force over
every positive BF16 max-abs for the power-of-two rule, block and row
permutation invariances.
"""

from fractions import Fraction

import numpy as np
import torch

import workloads
from oracle import e4m3, quant


def _tiny():
    return workloads.dense_inputs("tiny")


def _special_rows(K=512):
    """Rows with zero groups, BF16 subnormals, negative zeros, tiny amax."""
    rng = np.random.default_rng(5)
    rows = []
    r = np.zeros(K, np.float32)
    r[1::3] = -0.0
    rows.append(workloads.bf16_bits(r))                       # all +-0 groups
    r = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** -128)
    rows.append(workloads.bf16_bits(r))                       # subnormal/tiny amax
    r = rng.standard_normal(K).astype(np.float32)
    r[:128] *= np.float32(2.0 ** -133 / 4)                    # group 0 ~ tiny subnormals
    r[128:256] = np.float32(1e-37)                            # amax below 448/FLT_MAX
    rows.append(workloads.bf16_bits(r))
    bits = rng.integers(0, 65536, size=K, dtype=np.uint64).astype(np.uint16)
    f = quant.bf16_bits_to_f32(bits)
    bits[~np.isfinite(f)] = 0x3F80
    rows.append(bits)                                         # random BF16 bit patterns
    return np.stack(rows)


def _all_inputs():
    A, W = _tiny()
    return np.concatenate([A, _special_rows()], axis=0), W


def test_amax_maps_to_448_and_codes_bounded():
    A, _ = _all_inputs()
    q, s = quant.quantize_act(A)
    x = quant.bf16_bits_to_f32(A).reshape(A.shape[0], -1, 128)
    qg = q.reshape(q.shape[0], -1, 128)
    amax = np.abs(x).max(axis=2)
    live = s.T > 0
    idx = np.abs(x).argmax(axis=2)
    at_max = np.take_along_axis(qg, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all((at_max[live] & 0x7F) == 0x7E)
    dec = np.abs(e4m3.decode(q))
    assert np.all(dec <= 448)
    # flushed groups: only signed zeros, s = 0, and only when 448/amax overflows
    flushed = ~live
    assert np.all((qg[flushed] & 0x7F) == 0)
    with np.errstate(divide="ignore", over="ignore"):
        inv64 = 448.0 / amax.astype(np.float64)
    assert np.all(flushed == ((amax == 0) | (inv64 > np.finfo(np.float32).max * (1 + 2.0 ** -24))))
    assert flushed.any() and live.any()


def test_dequant_error_bound():
    A, _ = _all_inputs()
    q, s = quant.quantize_act(A)
    x = quant.bf16_bits_to_f32(A).astype(np.float64)
    xd = quant.dequantize_act(q, s)
    sfull = np.repeat(s.T.astype(np.float64), 128, axis=1)
    err = np.abs(x - xd)
    live = sfull > 0
    big = live & (np.abs(x) >= 2.0 ** -6 * sfull)
    assert np.all(err[big] <= (2.0 ** -4 + 2.0 ** -20) * np.abs(x[big]))
    small = live & ~big
    assert np.all(err[small] <= 2.0 ** -10 * sfull[small] + 2.0 ** -20 * np.abs(x[small]))


def test_matches_torch_float32_pipeline():
    """Independent arithmetic: torch float32 max/divide/multiply + float8 cast."""
    A, _ = _all_inputs()
    q, s = quant.quantize_act(A)
    x = torch.from_numpy(quant.bf16_bits_to_f32(A).copy()).reshape(A.shape[0], -1, 128)
    amax = x.abs().amax(dim=2, keepdim=True)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    fl = ~torch.isfinite(inv)
    inv = torch.where(fl, torch.zeros_like(inv), inv)
    ref_q = (x * inv).to(torch.float8_e4m3fn).view(torch.uint8).reshape(A.shape).numpy()
    ref_s = torch.where(fl, torch.zeros_like(amax), amax / 448.0)[:, :, 0].T.numpy()
    assert np.array_equal(q, ref_q)
    assert np.array_equal(s.view(np.uint32), np.ascontiguousarray(ref_s).view(np.uint32))


def test_scale_is_correctly_rounded_division():
    """s and inv are the RNE float32 of the exact quotients (checked with Fractions)."""
    A, _ = _tiny()
    _, s = quant.quantize_act(A)
    x = quant.bf16_bits_to_f32(A).reshape(A.shape[0], -1, 128)
    amax = np.abs(x).max(axis=2)
    for a, got in list(zip(amax.ravel(), s.T.ravel()))[:300]:
        exact = Fraction(float(a)) / 448
        lo = Fraction(float(np.float32(got)))
        # got is a float32 and no float32 lies strictly closer to the exact value
        up = Fraction(float(np.nextafter(np.float32(got), np.float32(np.inf))))
        dn = Fraction(float(np.nextafter(np.float32(got), np.float32(0))))
        assert abs(lo - exact) <= abs(up - exact) and abs(lo - exact) <= abs(dn - exact)


def test_quantize_commutes_with_row_gather():
    A, _ = _all_inputs()
    q, s = quant.quantize_act(A)
    perm = np.random.default_rng(3).permutation(A.shape[0])
    rows = np.concatenate([perm, perm[:7]])
    q2, s2 = quant.quantize_act(A[rows])
    assert np.array_equal(q2, q[rows]) and np.array_equal(s2, s[:, rows])


def test_weight_block_rules():
    _, W = _tiny()
    W = W.copy()
    W[128:256, 0:128] = 0  # one all-zero block
    q, s = quant.quantize_weight(W)
    assert s.shape == (2, 4)
    assert s[1, 0] == 0 and np.all((q[128:256, 0:128] & 0x7F) == 0)
    w = quant.bf16_bits_to_f32(W)
    for nb in range(2):
        for kb in range(4):
            blk = w[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            a = np.abs(blk).max()
            if a == 0:
                continue
            qb = q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert s[nb, kb] == np.float32(a / np.float32(448))
            i = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert (qb[i] & 0x7F) == 0x7E
    # block invariance: permuting elements inside a block keeps its scale
    blk = W[0:128, 128:256].copy().ravel()
    W2 = W.copy()
    W2[0:128, 128:256] = np.random.default_rng(1).permutation(blk).reshape(128, 128)
    _, s2 = quant.quantize_weight(W2)
    assert np.array_equal(s, s2)


def test_weight_dequant_error_bound():
    _, W = _tiny()
    q, s = quant.quantize_weight(W)
    w = quant.bf16_bits_to_f32(W)
    for nb in range(2):
        for kb in range(4):
            blk = w[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].astype(np.float64)
            dec = e4m3.decode(q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]) * float(s[nb, kb])
            assert np.all(np.abs(dec - blk) <= 2.0 ** -4 * np.abs(blk) + 2.0 ** -10 * float(s[nb, kb]))


def test_pow2_rule_bruteforce_all_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)  # every positive finite BF16
    a = (bits << 16).view(np.float32).astype(np.float64)
    e = quant.pow2_exponent(a)
    ok = 448.0 * np.ldexp(1.0, e) >= a
    prev_bad = 448.0 * np.ldexp(1.0, e - 1) < a
    assert np.all(ok) and np.all(prev_bad)
    # brute-force smallest e by search
    for ai, ei in list(zip(a, e))[::97]:
        k = -200
        while 448.0 * 2.0 ** k < ai:
            k += 1
        assert k == ei


def test_pow2_quantizer_invariants():
    A, _ = _all_inputs()
    q, s = quant.quantize_act(A, mode="pow2")
    x = quant.bf16_bits_to_f32(A).reshape(A.shape[0], -1, 128).astype(np.float64)
    amax = np.abs(x).max(axis=2).T
    live = amax > 0
    m, _ = np.frexp(s[live].astype(np.float64))
    assert np.all(m == 0.5), "scales must be powers of two"
    r = amax[live] / s[live].astype(np.float64)
    assert np.all((r > 224) & (r <= 448))
    assert np.all(s[~live] == 0)
    # exact scaling: x / s is representable and the code is its RNE encoding
    sfull = np.repeat(s.T.astype(np.float64), 128, axis=1).reshape(x.shape)
    y = np.where(sfull > 0, x / np.where(sfull > 0, sfull, 1), 0.0)
    for yi, xi, si in list(zip(y.ravel(), x.ravel(), sfull.ravel()))[::101]:
        if si > 0:
            assert Fraction(float(yi)) == Fraction(float(xi)) / Fraction(float(si))
    xd = quant.dequantize_act(q, s).reshape(x.shape)
    assert np.all(np.abs(xd - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * sfull)


def test_per_tensor_quantizer_outlier_sensitivity():
    """With outlier channels, one per-tensor scale pushes the small values of
    outlier-free groups into E4M3's subnormal range, while 1x128 groups keep
    them normal (the fine-grained quantization passage's motivation; a
    qualitative check on the tiny workload)."""
    A, _ = _tiny()
    x = quant.bf16_bits_to_f32(A).astype(np.float64)
    qf, sf = quant.quantize_act(A)
    qt, st = quant.quantize_tensor(A)
    err_f = np.abs(quant.dequantize_act(qf, sf) - x)
    err_t = np.abs(e4m3.decode(qt) * float(st) - x)
    outl = workloads.outlier_channels(512, 1001, None, 2)
    clean_groups = sorted(set(range(4)) - set(int(c) // 128 for c in outl))
    assert clean_groups, "the tiny workload leaves groups without outlier channels"
    mask = np.zeros(x.shape, bool)
    for g in clean_groups:
        mask[:, g * 128:(g + 1) * 128] = True
    small = mask & (np.abs(x) < 2.0 ** -6 * float(st)) & (x != 0)
    assert small.sum() > 50
    rel_f = (err_f[small] / np.abs(x[small])).mean()
    rel_t = (err_t[small] / np.abs(x[small])).mean()
    assert rel_f <= 2.0 ** -4 and rel_t > 3 * rel_f


def test_outlier_study_gemm_error_fine_grained_vs_per_tensor():
    """GEMM-level outlier sensitivity (an accuracy study; the pages print no
    magnitudes, so the numbers are parity unpinned and only their order is
    asserted).  Dense-workload rows (64 rows x 1024 weight rows, K = 7168) with
    its 72 outlier K-channels scaled by c; errors of the exact products of the
    dequantized operands against the exact BF16 product, in units of
    sum_k |a_k||w_k|, weights always 128x128-block quantized.  Without outliers
    one scale per tensor is as good as 1x128 groups; with them the per-tensor
    activation scale is worse by a quarter or more."""
    from oracle import gemm
    c = workloads.WORKLOADS["dense"]
    K = c["K"]
    outl = workloads.outlier_channels(K, c["seed"], c["outlier_frac"], c["outlier_count"])
    W = workloads.weight_rows(np.arange(1024), K, c["seed"], c["w_std"])
    qw, sw = quant.quantize_weight(W)
    Wd = quant.dequantize_weight(qw, sw)
    ratio = {}
    for mult in (1.0, 30.0, 300.0):
        A = workloads.act_rows(np.arange(64), K, c["seed"], c["act_std"], outl, mult)
        ref = gemm.gemm_bf16(A, W)
        absb = gemm.abs_bound_bf16(A, W)
        qa, sa = quant.quantize_act(A)
        ef = np.median(np.abs(quant.dequantize_act(qa, sa) @ Wd.T - ref) / absb)
        qt, st = quant.quantize_tensor(A)
        et = np.median(np.abs((e4m3.decode(qt) * float(st)) @ Wd.T - ref) / absb)
        ratio[mult] = et / ef
        print(f"outliers x{mult:g}: fine {ef:.3e} per-tensor {et:.3e} ratio {et / ef:.2f}")
        assert ef < 2e-3 if mult <= 30 else ef < 5e-3
    assert abs(ratio[1.0] - 1.0) < 0.03
    assert ratio[30.0] > 1.15 and ratio[300.0] > 1.2


def test_transposed_quantizers_are_the_rules_on_the_transpose():
    """quantize_act_t groups 128 consecutive rows of a column (its codes and
    scales equal a column-by-column evaluation of the 1x128 rule written out
    here); quantize_weight_t is quantize_weight with every block transposed."""
    rng = np.random.default_rng(9)
    M, K = 256, 384
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, 5] *= 40
    x[130, :] = 0
    xb = workloads.bf16_bits(x)
    qt, st = quant.quantize_act_t(xb)
    assert qt.shape == (K, M) and st.shape == (M // 128, K)
    xv = quant.bf16_bits_to_f32(xb)
    for k in (0, 5, 200, K - 1):
        for g in range(M // 128):
            col = xv[g * 128:(g + 1) * 128, k]
            amax = np.float32(np.abs(col).max())
            inv = np.float32(448.0) / amax
            assert st[g, k] == np.float32(amax / np.float32(448.0))
            want = e4m3.encode((col * inv).astype(np.float32))
            assert np.array_equal(qt[k, g * 128:(g + 1) * 128], want)
    # weights: the same 128x128 blocks, transposed
    w = workloads.bf16_bits((rng.standard_normal((256, 384)) * 0.02).astype(np.float32))
    q, s = quant.quantize_weight(w)
    qwt, swt = quant.quantize_weight_t(w)
    assert np.array_equal(qwt, q.T) and np.array_equal(swt, s.T)
    for mode in ("f32", "pow2"):
        q2, s2 = quant.quantize_weight(w, mode)
        q3, s3 = quant.quantize_weight_t(w, mode)
        assert np.array_equal(q3, q2.T) and np.array_equal(s3, s2.T)
