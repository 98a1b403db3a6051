"""GPU parity of the block-scaled GEMM (fp8q_gemm, fp8q_gemm_precise) and the
grouped GEMM (fp8q_grouped_gemm, fp8q_grouped_gemm_precise) against the CPU
oracle, through the C ABI.

Acceptance:
- the precise calls (gpu_util.assert_gemm_strict): |C_gpu - C_exact| <= 1e-5 *
  sum_k |a_k||b_k| (+ half a BF16 ulp of C_exact) on every checked output;
- the FP8-MFMA calls (gpu_util.assert_gemm_bounded): within the a-priori bound
  of the matrix core's 8-product truncation plus FP32 rounding, computed from
  the operands alone, on every checked output (the fraction within the 1e-5
  tolerance is reported).
The GPU operands come from the GPU quantizers; the oracle re-quantizes the
same BF16 inputs itself (the quantizers are bit-exact, checked separately).
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import (DEV, assert_gemm_bounded, assert_gemm_strict, bf16_to_bits, fq, host,
                      to_dev_bf16)
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


def _run_dense(A_bits, W_bits, out="f32", mode="f32", precise=False):
    f = fq()
    a = to_dev_bf16(A_bits)
    w = to_dev_bf16(W_bits)
    aq, as_ = f.quantize_act(a, mode)
    wq, ws = f.quantize_weight(w, mode)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = f.gemm(aq, as_, wq, ws, out_dtype=dt, precise=precise)
    torch.cuda.synchronize()
    return c


def _c_host(c):
    if c.dtype == torch.bfloat16:
        return c.float().cpu().numpy().astype(np.float64)
    return host(c)


def _oracle_q(A_bits, W_bits, mode="f32"):
    qa, sa = oquant.quantize_act(A_bits, mode)
    qw, sw = oquant.quantize_weight(W_bits, mode)
    return qa, sa, qw, sw


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["f32", "pow2"])
def test_gemm_tiny_full(out, mode):
    """The tiny workload (x50 outlier channels), every output: the FP8-MFMA
    call within its bound, the precise call within 1e-5 * sum|a||b|."""
    A, W = workloads.dense_inputs("tiny")
    q = _oracle_q(A, W, mode)
    c = _run_dense(A, W, out, mode)
    r = assert_gemm_bounded(_c_host(c), *q, out=out, what=f"tiny {out} {mode}", model_rows=8)
    cp = _run_dense(A, W, out, mode, precise=True)
    rp = assert_gemm_strict(_c_host(cp), *q, out=out, what=f"tiny precise {out} {mode}")
    print(f"tiny {out} {mode}: fp8 {r}; precise {rp}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 384, 640), (255, 256, 256),
                                   (300, 512, 1152), (513, 640, 384), (64, 128, 2048)])
def test_gemm_ragged_shapes(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = workloads.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    q = _oracle_q(A, W)
    assert_gemm_bounded(_c_host(_run_dense(A, W)), *q, what=f"{M}x{N}x{K}")
    assert_gemm_strict(_c_host(_run_dense(A, W, precise=True)), *q,
                       what=f"precise {M}x{N}x{K}")


def test_gemm_zero_groups_and_same_sign():
    """Flushed groups contribute zero; all-positive operands (no cancellation)
    stress the accumulation order."""
    rng = np.random.default_rng(4)
    M, N, K = 200, 256, 1024
    A = np.abs(rng.standard_normal((M, K))).astype(np.float32)
    A[:, 256:384] = 0
    A[7, :] = 0
    W = np.abs(rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[128:, 512:640] = 0
    A, W = workloads.bf16_bits(A), workloads.bf16_bits(W)
    c = _run_dense(A, W)
    ch = _c_host(c)
    assert np.all(ch[7] == 0)
    q = _oracle_q(A, W)
    assert_gemm_bounded(ch, *q, what="zero groups / same sign")
    cp = _c_host(_run_dense(A, W, precise=True))
    assert np.all(cp[7] == 0)
    assert_gemm_strict(cp, *q, what="precise zero groups / same sign")


def test_gemm_dense_full_size_sampled():
    """The dense 4096 x 4096 x 7168 workload in the bench's launch configuration;
    the oracle checks 48 sampled rows against every column (the FP8-MFMA
    call's truncation bound on 4 of the 32 weight blocks)."""
    cfg = workloads.WORKLOADS["dense"]
    A, W = workloads.dense_inputs("dense")
    f = fq()
    aq, as_ = f.quantize_act(to_dev_bf16(A))
    wq, ws = f.quantize_weight(to_dev_bf16(W))
    c = f.gemm(aq, as_, wq, ws)
    cp = f.gemm(aq, as_, wq, ws, precise=True)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(cfg["M"], 46, replace=False))
    rows = np.concatenate([[0], rows, [cfg["M"] - 1]])
    qa, sa = oquant.quantize_act(A[rows])
    qw, sw = oquant.quantize_weight(W)
    cols = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in (0, 9, 22, 31)])
    r = assert_gemm_bounded(_c_host(c)[rows], qa, sa, qw, sw, what="dense sampled",
                            bound_cols=cols)
    rp = assert_gemm_strict(_c_host(cp)[rows], qa, sa, qw, sw, what="dense precise sampled")
    print(f"dense: fp8 {r}; precise {rp}")


@pytest.mark.parametrize("precise", [False, True])
def test_gemm_determinism(precise):
    A, W = workloads.dense_inputs("tiny")
    c1 = _c_host(_run_dense(A, W, precise=precise))
    c2 = _c_host(_run_dense(A, W, precise=precise))
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


# ----------------------------------------------------------------- grouped
def _grouped_case(counts, N, K, seed, extra_rows=0):
    rng = np.random.default_rng(seed)
    G = len(counts)
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    Mt = int(off[-1]) + extra_rows
    A = workloads.bf16_bits(rng.standard_normal((Mt, K)).astype(np.float32))
    Ws = [workloads.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
          for _ in range(G)]
    return A, np.stack(Ws), off


def _run_grouped(A, Wst, off, out="f32", sentinel=None, precise=False):
    f = fq()
    G, N, K = Wst.shape
    a = to_dev_bf16(A)
    w = to_dev_bf16(Wst.reshape(G * N, K))
    aq, as_ = f.quantize_act(a)
    wq, ws = f.quantize_weight(w)
    wq = wq.view(G, N, K)
    ws = ws.view(G, N // 128, K // 128)
    d_off = torch.from_numpy(off).to(DEV)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = torch.full((A.shape[0], N), float("nan") if sentinel is None else sentinel,
                   dtype=dt, device=DEV)
    (f.fp8q_grouped_gemm_precise if precise else f.fp8q_grouped_gemm)(aq, as_, d_off, wq, ws, c)
    torch.cuda.synchronize()
    return c


def _check_grouped(c, A, Wst, off, experts, out="f32", max_rows=None, precise=False):
    ch = _c_host(c)
    qa, sa = oquant.quantize_act(A)
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        rows = np.arange(r0, r1)
        if max_rows and len(rows) > max_rows:
            rows = np.sort(np.random.default_rng(e).choice(rows, max_rows, replace=False))
        qw, sw = oquant.quantize_weight(Wst[e])
        if precise:
            assert_gemm_strict(ch[rows], qa[rows], sa[:, rows], qw, sw, out=out,
                               what=f"precise expert {e}")
        else:
            assert_gemm_bounded(ch[rows], qa[rows], sa[:, rows], qw, sw, out=out,
                                what=f"expert {e}")


def _assert_every_expert_equals_dense(c, cp, aq, as_, off, wq, ws, what):
    """Every row of a full-size grouped output, fast (c) and precise (cp), is
    bitwise equal to the dense GEMM of its expert's weights on that expert's
    rows: an output's arithmetic does not depend on the tile that computes it
    (one chunk partial per MFMA block, the same promotion order), so this
    carries the dense path's oracle checks to every output of the workload."""
    f = fq()
    bits = (lambda t: t.view(torch.int16)) if c.dtype == torch.bfloat16 else \
        (lambda t: t.view(torch.int32))
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        a_e, s_e = aq[lo:hi].contiguous(), as_[:, lo:hi].contiguous()
        ce = f.gemm(a_e, s_e, wq[e], ws[e], out_dtype=c.dtype)
        cpe = f.gemm(a_e, s_e, wq[e], ws[e], out_dtype=c.dtype, precise=True)
        torch.cuda.synchronize()
        assert torch.equal(bits(c[lo:hi]), bits(ce)), f"{what}: expert {e} differs from dense"
        assert torch.equal(bits(cp[lo:hi]), bits(cpe)), \
            f"{what}: precise expert {e} differs from dense"


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("precise", [False, True])
def test_grouped_small_with_empty_experts(out, precise):
    counts = [3, 0, 17, 1, 0, 260, 40]
    A, Wst, off = _grouped_case(counts, 256, 384, 11, extra_rows=5)
    c = _run_grouped(A, Wst, off, out, precise=precise)
    _check_grouped(c, A, Wst, off, range(len(counts)), out, precise=precise)
    tail = _c_host(c)[off[-1]:]
    assert np.all(np.isnan(tail)), "rows past off[G] must be left untouched"


@pytest.mark.parametrize("precise", [False, True])
def test_grouped_single_expert_equals_dense(precise):
    A, Wst, off = _grouped_case([300], 384, 640, 12)
    cg = _c_host(_run_grouped(A, Wst, off, precise=precise))
    cd = _c_host(_run_dense(A, Wst[0], precise=precise))
    assert np.array_equal(cg.view(np.uint32), cd.view(np.uint32))


def test_grouped_decode_workload_sampled():
    """Decode shape: 32 experts, M_e uniform in [16, 256], N 4096, K 7168, BF16
    out; expert weights drawn on the device, oracle on 4 sampled experts, and
    every expert's rows bitwise equal to the dense GEMM on them."""
    cfg = workloads.WORKLOADS["decode"]
    counts, off = workloads.decode_counts(cfg["experts"], cfg["m_lo"], cfg["m_hi"], cfg["seed"])
    G, N, K = cfg["experts"], cfg["N"], cfg["K"]
    outl = workloads.outlier_channels(K, cfg["seed"], cfg["outlier_frac"], cfg["outlier_count"])
    A = workloads.act_rows(np.arange(int(off[-1])), K, cfg["seed"], cfg["act_std"], outl,
                           cfg["outlier_mult"])
    f = fq()
    w = torch.empty((G, N, K), dtype=torch.bfloat16, device=DEV)
    for e in range(G):
        w[e] = workloads.expert_weight_torch(e, N, K, cfg["seed"], cfg["w_std"], DEV)
    aq, as_ = f.quantize_act(to_dev_bf16(A))
    wq, ws = f.quantize_weight(w.view(G * N, K))
    args = (aq, as_, torch.from_numpy(off).to(DEV), wq.view(G, N, K),
            ws.view(G, N // 128, K // 128))
    c = f.grouped_gemm(*args, out_dtype=torch.bfloat16)
    cp = f.grouped_gemm(*args, out_dtype=torch.bfloat16, precise=True)
    torch.cuda.synchronize()
    ch, chp = _c_host(c), _c_host(cp)
    qa, sa = oquant.quantize_act(A)
    cols = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in (3, 30)])
    for e in (0, 7, int(np.argmax(counts)), G - 1):
        Wb = bf16_to_bits(w[e])
        qw, sw = oquant.quantize_weight(Wb)
        assert np.array_equal(host(wq.view(G, N, K)[e]), qw)
        r0, r1 = int(off[e]), int(off[e + 1])
        rows = np.arange(r0, r1)
        if len(rows) > 24:
            rows = np.sort(np.random.default_rng(e).choice(rows, 24, replace=False))
        assert_gemm_bounded(ch[rows], qa[rows], sa[:, rows], qw, sw, out="bf16",
                            bound_cols=cols, what=f"decode expert {e}")
        assert_gemm_strict(chp[rows], qa[rows], sa[:, rows], qw, sw, out="bf16",
                           what=f"decode precise expert {e}")
    _assert_every_expert_equals_dense(c, cp, aq, as_, off, args[3], args[4], "decode")


@pytest.mark.parametrize("precise", [False, True])
def test_grouped_determinism_all_tile_configs(precise):
    """Repeated launches are bitwise identical, with experts of every staged
    row count (1..64, ..128, ..160, ..192, ..256 and multi-tile) so each
    grouped ring configuration runs with many tiles in flight.  150 and 160
    rows put live rows in the fourth row of 48-row waves of a 160-row tile."""
    counts = [1, 40, 64, 65, 128, 129, 150, 160, 161, 192, 193, 256, 300, 0, 77] * 3
    N, K = 256, 2048
    A, Wst, off = _grouped_case(counts, N, K, seed=21)
    runs = [host(_run_grouped(A, Wst, off, precise=precise)) for _ in range(4)]
    for r in runs[1:]:
        assert np.array_equal(r.view(np.uint32), runs[0].view(np.uint32))
    c0 = torch.from_numpy(runs[0])
    _check_grouped(c0, A, Wst, off, [1, 3, 5, 8, 11, 12], max_rows=24, precise=precise)
    # every row of the 150- and 160-row experts
    _check_grouped(c0, A, Wst, off, [6, 7], precise=precise)


def test_grouped_moe_workload_sampled():
    """MoE shape at full size: 4096 tokens routed top-8 over 256 experts
    (32768 gathered rows), N 4096, K 7168, FP32 out, in the launch bench.py
    times.  Weights are drawn on the device and quantized expert by expert;
    the oracle checks the codes of 4 sampled experts bit-exactly and their
    GEMM outputs on sampled rows, plus the activation codes of those rows;
    every expert's rows are bitwise equal to the dense GEMM on them."""
    cfg = workloads.WORKLOADS["moe"]
    G, N, K = cfg["experts"], cfg["N"], cfg["K"]
    counts, off, token_of = workloads.moe_routing(cfg["tokens"], G, cfg["topk"], cfg["seed"])
    assert int(off[-1]) == cfg["tokens"] * cfg["topk"]
    outl = workloads.outlier_channels(K, cfg["seed"], cfg["outlier_frac"], cfg["outlier_count"])
    tok = workloads.rows_threaded(workloads.act_rows, np.arange(cfg["tokens"]), K, cfg["seed"],
                                  cfg["act_std"], outl, cfg["outlier_mult"])
    A = tok[token_of]
    f = fq()
    wq = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    ws = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=DEV)
    for e in range(G):
        f.fp8q_quantize_weight(workloads.expert_weight_torch(e, N, K, cfg["seed"], cfg["w_std"],
                                                             DEV), wq[e], ws[e])
    aq, as_ = f.quantize_act(to_dev_bf16(A))
    c = torch.full((A.shape[0], N), float("nan"), dtype=torch.float32, device=DEV)
    f.fp8q_grouped_gemm(aq, as_, torch.from_numpy(off).to(DEV), wq, ws, c)
    cp = torch.full((A.shape[0], N), float("nan"), dtype=torch.float32, device=DEV)
    f.fp8q_grouped_gemm_precise(aq, as_, torch.from_numpy(off).to(DEV), wq, ws, cp)
    torch.cuda.synchronize()
    cols = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in (5, 26)])
    for e in (0, int(np.argmin(counts)), int(np.argmax(counts)), G - 1):
        Wb = bf16_to_bits(workloads.expert_weight_torch(e, N, K, cfg["seed"], cfg["w_std"], DEV))
        qw, sw = oquant.quantize_weight(Wb)
        assert np.array_equal(host(wq[e]), qw), f"expert {e} weight codes"
        assert np.array_equal(host(ws[e]).view(np.uint32), sw.view(np.uint32))
        r0, r1 = int(off[e]), int(off[e + 1])
        rows = np.arange(r0, r1)
        rows = np.sort(np.random.default_rng(e).choice(rows, min(16, len(rows)), replace=False))
        # quantization is row-wise, so the sampled rows quantize on their own
        qa, sa = oquant.quantize_act(A[rows])
        assert np.array_equal(host(aq[torch.from_numpy(rows).to(DEV)]), qa)
        assert np.array_equal(host(as_[:, torch.from_numpy(rows).to(DEV)]).view(np.uint32),
                              sa.view(np.uint32))
        ch = host(c[torch.from_numpy(rows).to(DEV)])
        assert_gemm_bounded(ch, qa, sa, qw, sw, bound_cols=cols, what=f"moe expert {e}")
        chp = host(cp[torch.from_numpy(rows).to(DEV)])
        assert_gemm_strict(chp, qa, sa, qw, sw, what=f"moe precise expert {e}")
    _assert_every_expert_equals_dense(c, cp, aq, as_, off, wq, ws, "moe")


@pytest.mark.parametrize("G", [1000, 1024])
@pytest.mark.parametrize("precise", [False, True])
def test_grouped_many_experts(G, precise):
    """Up to the 1024-expert limit: the device prefix scan runs over two
    512-expert chunks.  Most experts are empty; the others hold 1..70 rows,
    including the first and the last expert."""
    rng = np.random.default_rng(G)
    counts = np.where(rng.random(G) < 0.08, rng.integers(1, 71, G), 0)
    counts[0], counts[-1], counts[511], counts[512] = 3, 65, 1, 64
    N, K = 128, 256
    A, Wst, off = _grouped_case(list(counts), N, K, seed=G, extra_rows=3)
    c = _run_grouped(A, Wst, off, precise=precise)
    live = [e for e in range(G) if counts[e] > 0]
    _check_grouped(c, A, Wst, off, live, precise=precise)
    assert np.all(np.isnan(_c_host(c)[off[-1]:])), "rows past off[G] must be left untouched"
