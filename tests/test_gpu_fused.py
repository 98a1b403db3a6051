"""GPU parity of the GEMMs that quantize their BF16 activations themselves
(fp8q_gemm_fused, fp8q_grouped_gemm_fused), through the C ABI.

The fused cast applies fp8q_quantize_act's rule to the same groups and feeds
the same codes and scales to the same matrix-core sequence, so the bar is
bitwise equality with quantize-then-GEMM (fp8q_quantize_act followed by
fp8q_gemm / fp8q_grouped_gemm) on every output, in both scale modes; and,
directly, the FP8-MFMA GEMM bar of gpu_util.assert_gemm_bounded (the exact
oracle within the matrix core's truncation bound plus FP32 rounding) on
small cases.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import DEV, assert_gemm_bounded, fq, host, to_dev_bf16
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


def _bits(x):
    return workloads.bf16_bits(np.asarray(x, dtype=np.float32))


def _special(M, K, seed):
    """N(0,1) rows with an x40 outlier column, an all-zero 128-group (flushed
    in both modes), a group of BF16 subnormals only (flushed in the FP32 mode,
    a 2^-141-ish power-of-two scale in the other), and mixed-sign tiny values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, 5] *= 40
    if M > 3:
        x[3, :128] = 0
        x[2, -128:] = np.float32(2.0 ** -130) * rng.integers(-3, 4, size=128)
        x[1, 128:256] *= 1e-30 if K > 128 else 1.0
    return _bits(x)


def _same(c1, c2, what):
    a = c1.view(torch.int16 if c1.dtype == torch.bfloat16 else torch.int32)
    b = c2.view(torch.int16 if c2.dtype == torch.bfloat16 else torch.int32)
    bad = int((a != b).sum())
    assert bad == 0, f"{what}: {bad} outputs differ bitwise from quantize-then-GEMM"


def _weights(N, K, seed, mode="f32", G=None):
    rng = np.random.default_rng(seed)
    shape = (N, K) if G is None else (G * N, K)
    W = _bits(rng.standard_normal(shape) * 0.02)
    wq, ws = fq().quantize_weight(to_dev_bf16(W), mode)
    return W, wq, ws


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (2, 256, 256), (129, 128, 384), (17, 384, 640),
                                   (255, 256, 256), (300, 512, 1152), (513, 640, 384),
                                   (64, 128, 2048)])
@pytest.mark.parametrize("mode", ["f32", "pow2"])
def test_gemm_fused_equals_quantize_then_gemm(M, N, K, mode):
    """K = 128 and 256 take the paths where the chunk after next is clamped
    to the last chunk."""
    f = fq()
    X = _special(M, K, M * 3 + N + K)
    _, wq, ws = _weights(N, K, N + K, mode)
    x = to_dev_bf16(X)
    c = f.gemm_fused(x, wq, ws, mode)
    aq, as_ = f.quantize_act(x, mode)
    c_ref = f.gemm(aq, as_, wq, ws)
    torch.cuda.synchronize()
    _same(c, c_ref, f"{M}x{N}x{K} {mode}")


@pytest.mark.parametrize("mode", ["f32", "pow2"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_fused_against_oracle(mode, out):
    """The tiny workload plus the special groups, straight against the oracle."""
    M, N, K = 300, 256, 640
    X = _special(M, K, 77)
    W, wq, ws = _weights(N, K, 78, mode)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = fq().gemm_fused(to_dev_bf16(X), wq, ws, mode, out_dtype=dt)
    torch.cuda.synchronize()
    qa, sa = oquant.quantize_act(X, mode)
    qw, sw = oquant.quantize_weight(W, mode)
    assert np.array_equal(host(wq), qw)
    r = assert_gemm_bounded(c.float().cpu().numpy().astype(np.float64), qa, sa, qw, sw,
                            out=out, what=f"fused {mode} {out}", model_rows=4)
    print(f"fused {mode} {out}: {r}")


def test_gemm_fused_dense_workload_full_size():
    """4096 x 4096 x 7168 with the dense activation recipe, in the launch
    configuration bench.py times: every output bitwise equal to
    quantize-then-GEMM."""
    cfg = workloads.WORKLOADS["dense"]
    A, W = workloads.dense_inputs("dense")
    f = fq()
    x = to_dev_bf16(A)
    wq, ws = f.quantize_weight(to_dev_bf16(W))
    c = f.gemm_fused(x, wq, ws, out_dtype=torch.bfloat16)
    aq, as_ = f.quantize_act(x)
    c_ref = f.gemm(aq, as_, wq, ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert c.shape == (cfg["M"], cfg["N"])
    _same(c, c_ref, "dense workload")


# ----------------------------------------------------------------- grouped
def _grouped(counts, N, K, seed, mode, extra_rows=5, out="f32"):
    f = fq()
    G = len(counts)
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    X = _special(int(off[-1]) + extra_rows, K, seed)
    W, wq, ws = _weights(N, K, seed + 1, mode, G)
    x = to_dev_bf16(X)
    d_off = torch.from_numpy(off).to(DEV)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = torch.full((X.shape[0], N), float("nan"), dtype=dt, device=DEV)
    f.fp8q_grouped_gemm_fused(x, d_off, wq.view(G, N, K), ws.view(G, N // 128, K // 128), c,
                              mode)
    aq, as_ = f.quantize_act(x, mode)
    c_ref = torch.full_like(c, float("nan"))
    f.fp8q_grouped_gemm(aq, as_, d_off, wq.view(G, N, K), ws.view(G, N // 128, K // 128), c_ref)
    torch.cuda.synchronize()
    return X, W.reshape(G, N, K), off, c, c_ref


@pytest.mark.parametrize("mode", ["f32", "pow2"])
def test_grouped_fused_all_tile_configs(mode):
    """Experts of every staged row count (1..64, ..128, ..160, ..192, ..256 and
    several m-tiles), empty experts, and rows past off[G] left untouched."""
    counts = [3, 0, 17, 64, 65, 128, 129, 150, 160, 161, 192, 193, 256, 257, 600, 0, 40]
    X, Wst, off, c, c_ref = _grouped(counts, 256, 640, 31, mode)
    n = int(off[-1])
    _same(c[:n], c_ref[:n], f"grouped {mode}")
    assert torch.isnan(c[n:]).all(), "rows past off[G] must be left untouched"
    # straight against the oracle on a few experts (sampled rows)
    ch = host(c)
    qa, sa = oquant.quantize_act(X, mode)
    for e in (0, 2, 7, 13, 14):
        r0, r1 = int(off[e]), int(off[e + 1])
        rows = np.arange(r0, r1)
        if len(rows) > 24:
            rows = np.sort(np.random.default_rng(e).choice(rows, 24, replace=False))
        qw, sw = oquant.quantize_weight(Wst[e], mode)
        assert_gemm_bounded(ch[rows], qa[rows], sa[:, rows], qw, sw,
                            what=f"grouped fused {mode} expert {e}")


def test_grouped_fused_determinism_and_bf16_out():
    counts = [1, 40, 64, 65, 128, 129, 150, 160, 161, 192, 193, 256, 300, 0, 77] * 2
    runs = [_grouped(counts, 256, 1024, 41, "f32", out="bf16") for _ in range(3)]
    n = int(runs[0][2][-1])
    for r in runs:
        _same(r[3][:n], r[4][:n], "grouped bf16")
        _same(r[3][:n], runs[0][3][:n], "repeat")


def test_grouped_fused_decode_workload_full_size():
    """The decode workload (32 experts, M_e uniform in [16, 256], N 4096,
    K 7168, BF16 out) in the launch bench.py times: every output bitwise
    equal to quantize-then-GEMM."""
    cfg = workloads.WORKLOADS["decode"]
    counts, off = workloads.decode_counts(cfg["experts"], cfg["m_lo"], cfg["m_hi"], cfg["seed"])
    G, N, K = cfg["experts"], cfg["N"], cfg["K"]
    outl = workloads.outlier_channels(K, cfg["seed"], cfg["outlier_frac"], cfg["outlier_count"])
    A = workloads.act_rows(np.arange(int(off[-1])), K, cfg["seed"], cfg["act_std"], outl,
                           cfg["outlier_mult"])
    f = fq()
    wq = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    ws = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=DEV)
    for e in range(G):
        f.fp8q_quantize_weight(workloads.expert_weight_torch(e, N, K, cfg["seed"], cfg["w_std"],
                                                             DEV), wq[e], ws[e])
    x = to_dev_bf16(A)
    d_off = torch.from_numpy(off).to(DEV)
    c = f.grouped_gemm_fused(x, d_off, wq, ws, out_dtype=torch.bfloat16)
    aq, as_ = f.quantize_act(x)
    c_ref = f.grouped_gemm(aq, as_, d_off, wq, ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _same(c, c_ref, "decode workload")


def test_grouped_fused_many_experts():
    """1024 experts (the limit), most of them empty, the others 1..70 rows;
    one K chunk (K = 128), so every cast load past the first chunk is clamped."""
    rng = np.random.default_rng(1024)
    G = 1024
    counts = np.where(rng.random(G) < 0.08, rng.integers(1, 71, G), 0)
    counts[0], counts[-1], counts[511], counts[512] = 3, 65, 1, 64
    X, Wst, off, c, c_ref = _grouped(list(counts), 128, 128, 51, "f32", extra_rows=3)
    n = int(off[-1])
    _same(c[:n], c_ref[:n], "1024 experts")
    assert torch.isnan(c[n:]).all(), "rows past off[G] must be left untouched"


@pytest.mark.parametrize("mode", ["f32", "pow2"])
def test_gemm_fused_every_bf16_group_max(mode):
    """One activation group per positive finite BF16 value a (every subnormal
    and normal magnitude), holding a, -a/2 and small values: the fused cast's
    scale and codes for every possible group max, through the GEMM output,
    bitwise against quantize-then-GEMM."""
    a = np.arange(1, 0x7F80, dtype=np.uint16)
    groups = np.zeros((len(a), 128), np.uint16)
    groups[:, 0] = a
    groups[:, 1] = workloads.bf16_bits(-0.5 * oquant.bf16_bits_to_f32(a))
    groups[:, 2] = a >> 1  # a smaller positive bit pattern, so a smaller magnitude
    G = 8
    pad = (-len(a)) % G
    groups = np.concatenate([groups, np.zeros((pad, 128), np.uint16)])
    X = groups.reshape(-1, G * 128)
    f = fq()
    _, wq, ws = _weights(256, X.shape[1], 7, mode)
    x = to_dev_bf16(X)
    c = f.gemm_fused(x, wq, ws, mode)
    aq, as_ = f.quantize_act(x, mode)
    c_ref = f.gemm(aq, as_, wq, ws)
    torch.cuda.synchronize()
    _same(c, c_ref, f"every group max {mode}")
