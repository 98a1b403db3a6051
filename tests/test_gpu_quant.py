"""GPU parity of the quantizers: E4M3 bytes and FP32 scales bit-exact against
the CPU oracle, through the C ABI (fp8q_quantize_act / fp8q_quantize_weight)."""

import numpy as np
import pytest
import torch

import workloads
from oracle import quant as oquant
from gpu_util import fq, host, to_dev_bf16

pytestmark = pytest.mark.gpu


def _gpu_act(bits, mode):
    x = to_dev_bf16(bits)
    q, s = fq().quantize_act(x, mode)
    torch.cuda.synchronize()
    return host(q), host(s)


def _gpu_weight(bits, mode):
    w = to_dev_bf16(bits)
    q, s = fq().quantize_weight(w, mode)
    torch.cuda.synchronize()
    return host(q), host(s)


def _assert_same(gq, gs, rq, rs, what):
    if not np.array_equal(gq, rq):
        idx = np.argwhere(gq != rq)[0]
        raise AssertionError(f"{what}: codes differ at {tuple(idx)}: gpu {gq[tuple(idx)]:#04x} "
                             f"oracle {rq[tuple(idx)]:#04x} ({(gq != rq).sum()} bytes)")
    gb, rb = gs.view(np.uint32), rs.view(np.uint32)
    if not np.array_equal(gb, rb):
        idx = np.argwhere(gb != rb)[0]
        raise AssertionError(f"{what}: scales differ at {tuple(idx)}: gpu {gs[tuple(idx)]!r} "
                             f"oracle {rs[tuple(idx)]!r}")


def _special_rows(K):
    rng = np.random.default_rng(5)
    rows = []
    r = np.zeros(K, np.float32)
    r[1::3] = -0.0
    rows.append(workloads.bf16_bits(r))
    rows.append(workloads.bf16_bits(rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** -128)))
    r = rng.standard_normal(K).astype(np.float32)
    r[:128] *= np.float32(2.0 ** -135)
    r[128:256] = np.float32(1e-37)
    rows.append(workloads.bf16_bits(r))
    bits = rng.integers(0, 65536, size=K, dtype=np.uint64).astype(np.uint16)
    f = oquant.bf16_bits_to_f32(bits)
    bits[~np.isfinite(f)] = 0x3F80
    rows.append(bits)
    return np.stack(rows)


def _exhaustive_bf16_rows(amax_bits):
    """Every finite BF16 value with |v| <= the group max, 127 per group, each
    group's max element set to amax (so inv is fixed per row)."""
    amax = float(oquant.bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0])
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oquant.bf16_bits_to_f32(allb)
    vals = allb[np.isfinite(f) & (np.abs(f) <= amax)]
    n_groups = (len(vals) + 126) // 127
    pad = n_groups * 127 - len(vals)
    vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(n_groups, 127)
    groups = np.concatenate([np.full((n_groups, 1), amax_bits, np.uint16), vals], axis=1)
    G = 8
    n_rows = (n_groups + G - 1) // G
    extra = n_rows * G - n_groups
    groups = np.concatenate([groups, np.tile(groups[:1], (extra, 1))], axis=0)
    return groups.reshape(n_rows, G * 128)


@pytest.mark.parametrize("mode", ["f32", "pow2"])
def test_act_tiny_and_special(mode):
    A, _ = workloads.dense_inputs("tiny")
    bits = np.concatenate([A, _special_rows(512)], axis=0)
    gq, gs = _gpu_act(bits, mode)
    rq, rs = oquant.quantize_act(bits, mode)
    _assert_same(gq, gs, rq, rs, f"act tiny+special {mode}")


@pytest.mark.parametrize("M,K", [(1, 128), (17, 640), (300, 384), (33, 1280), (5, 128 * 9)])
def test_act_ragged_shapes(M, K):
    rng = np.random.default_rng(M * 1000 + K)
    bits = workloads.bf16_bits((rng.standard_normal((M, K)) * 3).astype(np.float32))
    for mode in ("f32", "pow2"):
        gq, gs = _gpu_act(bits, mode)
        rq, rs = oquant.quantize_act(bits, mode)
        _assert_same(gq, gs, rq, rs, f"act {M}x{K} {mode}")


@pytest.mark.parametrize("amax_bits", [0x43E0, 0x4360, 0x3F80, 0x4400, 0x3C00])
def test_act_exhaustive_bf16_values(amax_bits):
    """Every finite BF16 magnitude below the group max goes through the cast
    (448 -> inv 1; 224 -> inv 2; 1.0; 512; 2^-7), covering every E4M3
    rounding tie and subnormal output."""
    bits = _exhaustive_bf16_rows(amax_bits)
    for mode in ("f32", "pow2"):
        gq, gs = _gpu_act(bits, mode)
        rq, rs = oquant.quantize_act(bits, mode)
        _assert_same(gq, gs, rq, rs, f"act exhaustive amax={amax_bits:#06x} {mode}")


def test_act_every_bf16_group_max():
    """One group per positive finite BF16 value a (32,639 groups: every
    subnormal and normal magnitude), holding a, -a and zeros: the scale rule
    of both modes, including the exponent of subnormal maxima in the pow2
    mode, is checked for every possible group max."""
    a = np.arange(1, 0x7F80, dtype=np.uint16)          # 0x0001 .. 0x7F7F
    groups = np.zeros((len(a), 128), np.uint16)
    groups[:, 0] = a
    groups[:, 1] = a | 0x8000
    G = 8
    pad = (-len(a)) % G
    groups = np.concatenate([groups, np.zeros((pad, 128), np.uint16)])
    bits = groups.reshape(-1, G * 128)
    for mode in ("f32", "pow2"):
        gq, gs = _gpu_act(bits, mode)
        rq, rs = oquant.quantize_act(bits, mode)
        _assert_same(gq, gs, rq, rs, f"act every group max {mode}")


def test_act_random_bit_patterns():
    rng = np.random.default_rng(99)
    bits = rng.integers(0, 65536, size=(257, 1024), dtype=np.uint64).astype(np.uint16)
    f = oquant.bf16_bits_to_f32(bits)
    bits[~np.isfinite(f)] = 0
    for mode in ("f32", "pow2"):
        gq, gs = _gpu_act(bits, mode)
        rq, rs = oquant.quantize_act(bits, mode)
        _assert_same(gq, gs, rq, rs, f"act random bits {mode}")


def test_act_dense_full_size_sampled_rows():
    """The dense workload's 4096 x 7168 activation, quantized at full size in the
    bench's launch configuration; the oracle checks 96 sampled rows."""
    c = workloads.WORKLOADS["dense"]
    A, _ = workloads.dense_inputs("dense", rows_w=np.arange(0))
    gq, gs = _gpu_act(A, "f32")
    rows = np.random.default_rng(0).choice(c["M"], 96, replace=False)
    rows = np.concatenate([rows, [0, c["M"] - 1]])
    rq, rs = oquant.quantize_act(A[rows], "f32")
    _assert_same(gq[rows], gs[:, rows], rq, rs, "act dense sampled")


def test_act_determinism():
    A, _ = workloads.dense_inputs("tiny")
    a1 = _gpu_act(A, "f32")
    a2 = _gpu_act(A, "f32")
    assert np.array_equal(a1[0], a2[0]) and np.array_equal(a1[1], a2[1])


@pytest.mark.parametrize("mode", ["f32", "pow2"])
def test_weight_tiny_and_zero_block(mode):
    _, W = workloads.dense_inputs("tiny")
    W = W.copy()
    W[128:256, 0:128] = 0
    W[0:128, 256:384] = workloads.bf16_bits(np.full((128, 128), 1e-37, np.float32))
    gq, gs = _gpu_weight(W, mode)
    rq, rs = oquant.quantize_weight(W, mode)
    _assert_same(gq, gs, rq, rs, f"weight tiny {mode}")


@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (128, 128 * 11)])
def test_weight_ragged_shapes(N, K):
    rng = np.random.default_rng(N + K)
    bits = rng.integers(0, 65536, size=(N, K), dtype=np.uint64).astype(np.uint16)
    f = oquant.bf16_bits_to_f32(bits)
    bits[~np.isfinite(f)] = 0x4000
    for mode in ("f32", "pow2"):
        gq, gs = _gpu_weight(bits, mode)
        rq, rs = oquant.quantize_weight(bits, mode)
        _assert_same(gq, gs, rq, rs, f"weight {N}x{K} {mode}")


def test_weight_dense_full_size_sampled_blocks():
    c = workloads.WORKLOADS["dense"]
    _, W = workloads.dense_inputs("dense", rows_a=np.arange(0))
    gq, gs = _gpu_weight(W, "f32")
    for nb in (0, 13, c["N"] // 128 - 1):
        rows = slice(nb * 128, (nb + 1) * 128)
        rq, rs = oquant.quantize_weight(W[rows], "f32")
        _assert_same(gq[rows], gs[nb:nb + 1], rq, rs, f"weight dense block row {nb}")


def test_act_cast_sweep_every_bf16_against_128_group_maxima():
    """The hardware FP32 -> E4M3 conversion inside fp8q_quantize_act against
    oracle.e4m3.encode on a dense sweep of its inputs fl32(x * fl32(448 / a)):
    every finite BF16 x with |x| <= a (both signs, subnormals included)
    against each of the 128 BF16 group maxima a in [1, 2) (every BF16
    mantissa, so inv takes 128 different significands).  The sweep puts
    thousands of inputs within one FP32 ulp of E4M3 rounding midpoints (ties
    and their neighbours), in the normal and the subnormal E4M3 range."""
    maxima = np.arange(0x3F80, 0x4000, dtype=np.uint16)
    blocks = [_exhaustive_bf16_rows(int(a)) for a in maxima]
    bits = np.concatenate(blocks, axis=0)
    gq, gs = _gpu_act(bits, "f32")
    rq, rs = oquant.quantize_act(bits, "f32")
    _assert_same(gq, gs, rq, rs, "act cast sweep over 128 group maxima")
    # coverage: inputs of the cast within one FP32 ulp of an E4M3 midpoint
    from oracle import e4m3
    x = oquant.bf16_bits_to_f32(bits).reshape(bits.shape[0], -1, 128)
    inv = np.float32(448.0) / np.abs(x[:, :, :1])
    v = np.abs((x * inv).astype(np.float32)).ravel()
    pos = np.sort(e4m3.DECODE_TABLE[:0x7F].astype(np.float64))
    mids = (pos[1:] + pos[:-1]) / 2
    j = np.clip(np.searchsorted(mids, v), 1, len(mids) - 1)
    d = np.minimum(np.abs(v - mids[j]), np.abs(v - mids[j - 1]))
    near = int(np.sum(d <= np.spacing(v.astype(np.float32)).astype(np.float64)))
    print(f"cast sweep: {v.size} inputs, {near} within one FP32 ulp of a midpoint")
    assert near > 1000
