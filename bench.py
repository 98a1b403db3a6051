"""Benchmark of the fine-grained block-scaled FP8 hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  dense (default): 1x128 activation quantization of A [4096][7168] (BF16),
                   128x128 weight-block quantization of W [4096][7168] (BF16),
                   block-scaled FP8 GEMM with FP32 promotion every 128 K -> C FP32.
  moe:             activation quantization of the 32768 routed rows (4096 tokens
                   x top-8 of 256 experts) + grouped GEMM over the 256 experts'
                   pre-quantized weights (4096 x 7168 each).
  decode:          activation quantization of ~4352 rows + grouped GEMM over 32
                   experts (M_e uniform in [16, 256]), BF16 output.
  largek:          activation + weight quantization of 8192 x 65536 each + GEMM.
  backward:        the backward GEMMs of the dense layer (4096 tokens, N 4096,
                   K 7168) in FP8: Dgrad = 1x128 quantization of dY, transposed
                   weight quantization, block-scaled GEMM dX = dY W; Wgrad =
                   transposed (128-token) quantization of dY and X, GEMM with
                   row-group scales on both operands dW = dY^T X.  FP32 outputs.
  dense_fused,     the activation quantization fused into the GEMM (the FP8 cast
  decode_fused:    during the transfer the pages ask for): the same steps with
                   fp8q_gemm_fused / fp8q_grouped_gemm_fused in place of
                   fp8q_quantize_act + the GEMM; both are timed per kernel.
  bf16:            the comparison the pages' speed claim calls for: the BF16 GEMM
                   of the same kernel family on the dense shape (BF16 A and W,
                   FP32 out); the FP8 GEMM on the same inputs, quantized once,
                   and hipBLASLt's BF16 matmul (torch.matmul) are timed beside it.

Inputs are resident in HBM before the timed region; several input sets are
rotated so that every step streams its inputs from HBM rather than from the
256 MiB last-level cache.  Per-kernel durations come from HIP events recorded
on the stream the kernels are launched on (torch's current stream).

Prints ONE JSON line (rank 0).  ``--gpus`` above 1 is refused: this build runs
on one GPU.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s (% FP8 MFMA peak); quantize GB/s (% HBM)"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
METRIC_BF16 = "BF16 GEMM TFLOP/s (% BF16 MFMA peak), the reference of the FP8 path"

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
ACT_BYTES_PER_ELEM = 2 + 1 + 4 / 128          # BF16 in, E4M3 out, one FP32 scale per 128
WEIGHT_BYTES_PER_ELEM = 2 + 1 + 4 / 16384     # one FP32 scale per 128x128 block


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dense",
                   choices=["dense", "moe", "decode", "largek", "bf16", "backward", "dense_fused",
                            "decode_fused"])
    p.add_argument("--sets", type=int, default=0, help="input sets rotated (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (3 times): the known-size "
                        "kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def copy_probe(mib):
    import torch
    n = mib * 1024 * 1024 // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 4, "launches": 3}))


def gemm_bytes(M, N, K, out_bytes):
    return M * K * (1 + 4 / 128) + N * K * (1 + 4 / 16384) + M * N * out_bytes


# --------------------------------------------------------------------- setup
def setup_dense(fq, torch, name, sets, fused=False):
    import workloads
    c = workloads.WORKLOADS[name]
    M, N, K = c["M"], c["N"], c["K"]
    dev = "cuda:0"
    A_bits, W_bits = workloads.dense_inputs(name)
    A0 = torch.from_numpy(A_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    W0 = torch.from_numpy(W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    del A_bits, W_bits
    bufs = []
    for i in range(sets):
        A = A0 if i == 0 else A0.clone()
        W = W0 if i == 0 else W0.clone()
        aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        as_ = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
        wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        bufs.append((A, W, aq, as_, wq, ws, C))

    def launch(name, i):
        A, W, aq, as_, wq, ws, C = bufs[i % sets]
        if name == "fp8q_quantize_act":
            fq.fp8q_quantize_act(A, aq, as_)
        elif name == "fp8q_quantize_weight":
            fq.fp8q_quantize_weight(W, wq, ws)
        elif name == "fp8q_gemm_fused":
            fq.fp8q_gemm_fused(A, wq, ws, C)
        else:
            fq.fp8q_gemm(aq, as_, wq, ws, C)

    order = (["fp8q_quantize_weight", "fp8q_gemm_fused"] if fused else
             ["fp8q_quantize_act", "fp8q_quantize_weight", "fp8q_gemm"])

    def step(i):
        for name in order:
            launch(name, i)

    kernels = [
        ("fp8q_quantize_act", "hbm", M * K * ACT_BYTES_PER_ELEM, "B"),
        ("fp8q_quantize_weight", "hbm", N * K * WEIGHT_BYTES_PER_ELEM, "B"),
        ("fp8q_gemm", "mfma", 2.0 * M * N * K, "flop"),
    ]
    if fused:
        kernels.insert(0, ("fp8q_gemm_fused", "mfma", 2.0 * M * N * K, "flop"))
    flops = 2.0 * M * N * K
    tag = name + ("_fused" if fused else "")
    how = "quantized inside the GEMM" if fused else "1x128 act quant"
    cfg = {"workload": f"{tag}: A {M}x{K} bf16 ({how}), W {N}x{K} bf16 "
                       f"(128x128 block quant), C = A W^T fp32",
           "M": M, "N": N, "K": K, "out": "f32", "input_sets": sets}
    return step, launch, kernels, flops, cfg


def setup_bf16(fq, torch, sets):
    import workloads
    c = workloads.WORKLOADS["dense"]
    M, N, K = c["M"], c["N"], c["K"]
    dev = "cuda:0"
    A_bits, W_bits = workloads.dense_inputs("dense")
    A0 = torch.from_numpy(A_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    W0 = torch.from_numpy(W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    del A_bits, W_bits
    bufs = []
    for i in range(sets):
        A = A0 if i == 0 else A0.clone()
        W = W0 if i == 0 else W0.clone()
        Wt = W.t().contiguous()  # [K][N] for torch.matmul (no transposed views)
        aq, as_ = fq.quantize_act(A)
        wq, ws = fq.quantize_weight(W)
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        Cb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        bufs.append((A, W, Wt, aq, as_, wq, ws, C, Cb))

    def launch(name, i):
        A, W, Wt, aq, as_, wq, ws, C, Cb = bufs[i % sets]
        if name == "fp8q_gemm_bf16":
            fq.fp8q_gemm_bf16(A, W, C)
        elif name == "fp8q_gemm":
            fq.fp8q_gemm(aq, as_, wq, ws, C)
        else:  # hipBLASLt through torch, BF16 out
            torch.matmul(A, Wt, out=Cb)

    def step(i):
        launch("fp8q_gemm_bf16", i)

    flops = 2.0 * M * N * K
    kernels = [
        ("fp8q_gemm_bf16", "mfma_bf16", flops, "flop"),
        ("torch_matmul_bf16_hipblaslt", "mfma_bf16", flops, "flop"),
        ("fp8q_gemm", "mfma", flops, "flop"),
    ]
    cfg = {"workload": f"bf16: A {M}x{K} bf16, W {N}x{K} bf16, C = A W^T fp32 (BF16 GEMM of "
                       f"the FP8 kernel family; the dense workload's inputs)",
           "M": M, "N": N, "K": K, "out": "f32", "input_sets": sets}
    return step, launch, kernels, flops, cfg


def setup_backward(fq, torch, sets):
    import workloads
    c = workloads.WORKLOADS["dense"]
    M, N, K = c["M"], c["N"], c["K"]
    dev = "cuda:0"
    X_bits, W_bits = workloads.dense_inputs("dense")
    dY_bits = workloads.bf16_bits(
        (np.random.default_rng(c["seed"] + 7).standard_normal((M, N)) * 1e-2).astype(np.float32))
    to = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
    X0, W0, dY0 = to(X_bits), to(W_bits), to(dY_bits)
    del X_bits, W_bits, dY_bits
    f32, u8 = torch.float32, torch.uint8
    bufs = []
    for i in range(sets):
        X = X0 if i == 0 else X0.clone()
        W = W0 if i == 0 else W0.clone()
        dY = dY0 if i == 0 else dY0.clone()
        b = dict(X=X, W=W, dY=dY,
                 qd=torch.empty((M, N), dtype=u8, device=dev),
                 sd=torch.empty((N // 128, M), dtype=f32, device=dev),
                 qwt=torch.empty((K, N), dtype=u8, device=dev),
                 swt=torch.empty((K // 128, N // 128), dtype=f32, device=dev),
                 dX=torch.empty((M, K), dtype=f32, device=dev),
                 qdt=torch.empty((N, M), dtype=u8, device=dev),
                 sdt=torch.empty((M // 128, N), dtype=f32, device=dev),
                 qxt=torch.empty((K, M), dtype=u8, device=dev),
                 sxt=torch.empty((M // 128, K), dtype=f32, device=dev),
                 dW=torch.empty((N, K), dtype=f32, device=dev))
        bufs.append(b)

    def launch(name, i):
        b = bufs[i % sets]
        if name == "fp8q_quantize_act":
            fq.fp8q_quantize_act(b["dY"], b["qd"], b["sd"])
        elif name == "fp8q_quantize_weight_t":
            fq.fp8q_quantize_weight_t(b["W"], b["qwt"], b["swt"])
        elif name == "fp8q_gemm":
            fq.fp8q_gemm(b["qd"], b["sd"], b["qwt"], b["swt"], b["dX"])
        elif name == "fp8q_quantize_act_t:dY":
            fq.fp8q_quantize_act_t(b["dY"], b["qdt"], b["sdt"])
        elif name == "fp8q_quantize_act_t:X":
            fq.fp8q_quantize_act_t(b["X"], b["qxt"], b["sxt"])
        else:
            fq.fp8q_gemm_rowscaled(b["qdt"], b["sdt"], b["qxt"], b["sxt"], b["dW"])

    order = ["fp8q_quantize_act", "fp8q_quantize_weight_t", "fp8q_gemm",
             "fp8q_quantize_act_t:dY", "fp8q_quantize_act_t:X", "fp8q_gemm_rowscaled"]

    def step(i):
        for name in order:
            launch(name, i)

    g = 2.0 * M * N * K
    kernels = [
        ("fp8q_quantize_act", "hbm", M * N * ACT_BYTES_PER_ELEM, "B"),
        ("fp8q_quantize_weight_t", "hbm", N * K * WEIGHT_BYTES_PER_ELEM, "B"),
        ("fp8q_gemm", "mfma", g, "flop"),
        ("fp8q_quantize_act_t:dY", "hbm", M * N * ACT_BYTES_PER_ELEM, "B"),
        ("fp8q_quantize_act_t:X", "hbm", M * K * ACT_BYTES_PER_ELEM, "B"),
        ("fp8q_gemm_rowscaled", "mfma", g, "flop"),
    ]
    cfg = {"workload": f"backward: tokens {M}, N {N}, K {K}; Dgrad dX = dY W (1x128 quant of dY, "
                       f"transposed 128x128 quant of W, block-scaled GEMM) + Wgrad dW = dY^T X "
                       f"(128-token quant of dY and X, row-scaled GEMM), fp32 out",
           "M": M, "N": N, "K": K, "out": "f32", "input_sets": sets}
    return step, launch, kernels, 2 * g, cfg


def setup_grouped(fq, torch, name, sets, fused=False):
    import workloads
    c = workloads.WORKLOADS[name]
    dev = "cuda:0"
    N, K = c["N"], c["K"]
    if name == "moe":
        counts, off, token_of = workloads.moe_routing(c["tokens"], c["experts"], c["topk"], c["seed"])
        G = c["experts"]
        outl = workloads.outlier_channels(K, c["seed"], c["outlier_frac"], c["outlier_count"])
        tok = workloads.act_rows(np.arange(c["tokens"]), K, c["seed"], c["act_std"], outl,
                                 c["outlier_mult"])
        A_bits = tok[token_of]  # rows grouped by expert (the dispatch gather, untimed)
        out_dtype = torch.float32
    else:
        counts, off = workloads.decode_counts(c["experts"], c["m_lo"], c["m_hi"], c["seed"])
        G = c["experts"]
        outl = workloads.outlier_channels(K, c["seed"], c["outlier_frac"], c["outlier_count"])
        A_bits = workloads.act_rows(np.arange(int(off[-1])), K, c["seed"], c["act_std"], outl,
                                    c["outlier_mult"])
        out_dtype = torch.bfloat16
    Mt = int(off[-1])
    A0 = torch.from_numpy(A_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    del A_bits
    # expert weights: drawn on the device, quantized once (pre-quantized weights)
    wq = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=dev)
    for e in range(G):
        w = workloads.expert_weight_torch(e, N, K, c["seed"], c["w_std"], dev)
        fq.fp8q_quantize_weight(w, wq[e], ws[e])
    del w
    d_off = torch.from_numpy(off).to(dev)
    bufs = []
    for i in range(sets):
        A = A0 if i == 0 else A0.clone()
        aq = torch.empty((Mt, K), dtype=torch.uint8, device=dev)
        as_ = torch.empty((K // 128, Mt), dtype=torch.float32, device=dev)
        C = torch.empty((Mt, N), dtype=out_dtype, device=dev)
        bufs.append((A, aq, as_, C))

    def launch(name, i):
        A, aq, as_, C = bufs[i % sets]
        if name == "fp8q_quantize_act":
            fq.fp8q_quantize_act(A, aq, as_)
        elif name == "fp8q_grouped_gemm_fused":
            fq.fp8q_grouped_gemm_fused(A, d_off, wq, ws, C)
        else:
            fq.fp8q_grouped_gemm(aq, as_, d_off, wq, ws, C)

    def step(i):
        if fused:
            launch("fp8q_grouped_gemm_fused", i)
        else:
            launch("fp8q_quantize_act", i)
            launch("fp8q_grouped_gemm", i)

    ob = 2 if out_dtype == torch.bfloat16 else 4
    flops = 2.0 * Mt * N * K
    gbytes = G * N * K * (1 + 4 / 16384) + Mt * K * (1 + 4 / 128) + Mt * N * ob
    kernels = [
        ("fp8q_quantize_act", "hbm", Mt * K * ACT_BYTES_PER_ELEM, "B"),
        ("fp8q_grouped_gemm", "hbm", gbytes, "B"),
    ]
    if fused:
        # weights and their scales once, the BF16 activations once, the output
        fbytes = G * N * K * (1 + 4 / 16384) + Mt * K * 2 + Mt * N * ob
        kernels.insert(0, ("fp8q_grouped_gemm_fused", "hbm", fbytes, "B"))
    tag = name + ("_fused" if fused else "")
    how = ("grouped GEMM quantizing its BF16 activations (1x128) inside" if fused else
           "1x128 act quant + grouped GEMM")
    cfg = {"workload": f"{tag}: {G} experts, rows {Mt} (M_e {int(counts.min())}..{int(counts.max())}), "
                       f"N {N}, K {K}, {how}, weights pre-quantized 128x128",
           "experts": G, "rows": Mt, "N": N, "K": K, "out": "bf16" if ob == 2 else "f32",
           "input_sets": sets}
    return step, launch, kernels, flops, cfg


# -------------------------------------------------------- recorded traffic
GEMM_SOURCES = ("gemm_kernels.hip", "gemm_common.hpp", "fp8q_device.hpp", "quant_rules.hpp")


def kernel_source_digest():
    """sha256 over the code of the GEMM kernels' sources (in GEMM_SOURCES
    order, with comments and whitespace removed): traffic figures recorded
    under profiles/ are reported only while that code is unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        text = open(os.path.join(ROOT, "fine_grained_block_fp8q_amd", "csrc", name)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()


def recorded_traffic(kernel, cfg):
    """HBM-side bytes per launch from the committed rocprofv3 --pmc summary
    (FETCH_SIZE and WRITE_SIZE, calibrated on a copy of known size), or None
    if there is none for this kernel and workload or the kernel changed."""
    import glob
    digest = kernel_source_digest()
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        rec = {}
        for line in open(path):
            if line.startswith("traffic-record:"):
                for kv in line.split(":", 1)[1].split():
                    k, v = kv.split("=", 1)
                    rec[k] = v
        if (rec.get("kernel") == kernel and rec.get("workload") == cfg["workload"].split(":")[0]
                and rec.get("source_sha256") == digest):
            return float(rec["bytes_per_launch"])
    return None


# --------------------------------------------------------------- cpu baseline
def cpu_baseline(name):
    """The oracle, untuned, on a bounded sample of the workload (host cores):
    the whole dense workload (about 10-20 s), or for the other workloads a
    row sample whose flops scale the rate."""
    import workloads
    from oracle import gemm as ogemm, quant as oquant
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    if name == "backward":
        c = workloads.WORKLOADS["dense"]
        M, N, K = c["M"], c["N"], c["K"]
        rows = 256
        X, _ = workloads.dense_inputs("dense", rows_w=np.arange(128))
        dY = workloads.bf16_bits(
            (np.random.default_rng(c["seed"] + 7).standard_normal((M, N)) * 1e-2).astype(np.float32))
        t0 = time.perf_counter()
        qdt, sdt = oquant.quantize_act_t(dY)
        qxt, sxt = oquant.quantize_act_t(X)
        ogemm.gemm_rowscaled(qdt[:rows], sdt[:, :rows], qxt, sxt)
        dt = time.perf_counter() - t0
        flops = 2.0 * rows * K * M
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
                "sample": f"Wgrad rows 0..{rows - 1} of dW: oracle quantize_act_t of dY ({M}x{N}) "
                          f"and X ({M}x{K}) + exact row-scaled GEMM {rows}x{K}x{M}; {dt:.1f} s wall; "
                          f"value = 2*{rows}*{K}*{M} / wall"}
    if name == "bf16":
        c = workloads.WORKLOADS["dense"]
        M, N, K = c["M"], c["N"], c["K"]
        A, W = workloads.dense_inputs("dense")
        t0 = time.perf_counter()
        ogemm.gemm_bf16(A, W)
        dt = time.perf_counter() - t0
        return {"value": 2.0 * M * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores),
                "kind": "oracle",
                "sample": f"the whole bf16 workload: oracle gemm_bf16 (float64 matmul of "
                          f"the BF16 values) {M}x{N}x{K}; {dt:.1f} s wall; "
                          f"value = 2*M*N*K / wall"}
    c = workloads.WORKLOADS[name]
    if name == "dense":
        M, N, K = c["M"], c["N"], c["K"]
        A, W = workloads.dense_inputs(name)
        what = "the whole dense workload"
    elif name == "largek":
        M, N, K = 64, 512, c["K"]
        A, W = workloads.dense_inputs(name, rows_a=np.arange(M), rows_w=np.arange(N))
        what = f"rows 0..{M - 1} of A and 0..{N - 1} of W"
    else:
        M, N, K = 256, c["N"], c["K"]
        outl = workloads.outlier_channels(K, c["seed"], c["outlier_frac"], c["outlier_count"])
        A = workloads.act_rows(np.arange(M), K, c["seed"], c["act_std"], outl, c["outlier_mult"])
        W = workloads.weight_rows(np.arange(N), K, c["seed"], c["w_std"])
        what = f"{M} activation rows x one expert's {N}x{K} weight"
    t0 = time.perf_counter()
    qa, sa = oquant.quantize_act(A)
    qw, sw = oquant.quantize_weight(W)
    ogemm.gemm(qa, sa, qw, sw)
    dt = time.perf_counter() - t0
    flops = 2.0 * M * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{what}: oracle quantize_act({M}x{K}) + quantize_weight({N}x{K}) + exact "
                      f"float64 per-chunk GEMM {M}x{N}x{K}; {dt:.1f} s wall; value = 2*M*N*K / wall"}


# ----------------------------------------------------------------------- main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    import torch
    import fine_grained_block_fp8q_amd as fq

    sets = args.sets or (4 if args.workload in ("dense", "bf16", "dense_fused") else
                         2 if args.workload in ("decode", "backward", "decode_fused") else 1)
    base = args.workload.replace("_fused", "")
    fused = base != args.workload
    if base in ("dense", "largek"):
        step, launch, kernels, flops, cfg = setup_dense(fq, torch, base, sets, fused)
    elif args.workload == "bf16":
        step, launch, kernels, flops, cfg = setup_bf16(fq, torch, sets)
    elif args.workload == "backward":
        step, launch, kernels, flops, cfg = setup_backward(fq, torch, sets)
    else:
        step, launch, kernels, flops, cfg = setup_grouped(fq, torch, base, sets, fused)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, synchronized on both sides.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Per-kernel durations: HIP events on the launch stream around `steps`
    # back-to-back launches of each kernel (same inputs, same launch shape);
    # then the same launches once more, each with its own event pair, for the
    # median and the 10th / 90th percentiles.
    kout = {}
    for kname, bound, work, unit in kernels:
        launch(kname, 0)  # first call of a library kernel includes its set-up
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            launch(kname, args.warmup + i)
        e1.record()
        torch.cuda.synchronize()
        avg_ms = e0.elapsed_time(e1) / args.steps
        # Spread: one event pair per launch (the same launches again).
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        for i, (a, b) in enumerate(pairs):
            a.record()
            launch(kname, args.warmup + i)
            b.record()
        torch.cuda.synchronize()
        each = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
        spread = {"median_us": float(np.median(each)), "p10_us": float(np.percentile(each, 10)),
                  "p90_us": float(np.percentile(each, 90))}
        if unit == "B":
            ach = work / (avg_ms * 1e-3) / 1e9
            kout[kname] = {"avg_us": avg_ms * 1e3, "GB_s": ach, "frac_hbm": ach / PEAK_HBM_GBS,
                           "bytes": work, **spread}
        else:
            ach = work / (avg_ms * 1e-3) / 1e12
            peak_key, peak = (("frac_bf16_peak", PEAK_BF16_TFLOPS) if bound == "mfma_bf16"
                              else ("frac_fp8_peak", PEAK_FP8_TFLOPS))
            kout[kname] = {"avg_us": avg_ms * 1e3, "TFLOP_s": ach, peak_key: ach / peak,
                           "flops": work, **spread}

    if args.workload == "bf16":
        dom = kout["fp8q_gemm_bf16"]
        roof = {"kernel": "fp8q_gemm_bf16", "bound": "mfma", "achieved": dom["TFLOP_s"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": dom["TFLOP_s"] / PEAK_BF16_TFLOPS,
                "traffic": recorded_traffic("fp8q_gemm_bf16", cfg)}
        # The pages' claim, measured: FP8 GEMM speed over BF16 GEMM speed.
        roof["fp8_speedup_over_bf16"] = {
            "same_kernel_family": dom["avg_us"] / kout["fp8q_gemm"]["avg_us"],
            "hipblaslt_bf16_out": (kout["torch_matmul_bf16_hipblaslt"]["avg_us"]
                                   / kout["fp8q_gemm"]["avg_us"])}
    elif args.workload == "backward":
        dom = kout["fp8q_gemm_rowscaled"]
        roof = {"kernel": "fp8q_gemm_rowscaled", "bound": "mfma", "achieved": dom["TFLOP_s"],
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": dom["TFLOP_s"] / PEAK_FP8_TFLOPS,
                "traffic": recorded_traffic("fp8q_gemm_rowscaled", cfg)}
    elif args.workload == "dense_fused":
        dom = kout["fp8q_gemm_fused"]
        roof = {"kernel": "fp8q_gemm_fused", "bound": "mfma", "achieved": dom["TFLOP_s"],
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": dom["TFLOP_s"] / PEAK_FP8_TFLOPS,
                "traffic": recorded_traffic("fp8q_gemm_fused", cfg),
                "fused_vs_separate_us": {
                    "fused": dom["avg_us"],
                    "quantize_act_plus_gemm": (kout["fp8q_quantize_act"]["avg_us"]
                                               + kout["fp8q_gemm"]["avg_us"])}}
    elif args.workload == "decode_fused":
        dom = kout["fp8q_grouped_gemm_fused"]
        dom["TFLOP_s"] = flops / (dom["avg_us"] * 1e-6) / 1e12
        dom["frac_fp8_peak"] = dom["TFLOP_s"] / PEAK_FP8_TFLOPS
        roof = {"kernel": "fp8q_grouped_gemm_fused", "bound": "hbm", "achieved": dom["GB_s"],
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dom["GB_s"] / PEAK_HBM_GBS,
                "traffic": recorded_traffic("fp8q_grouped_gemm_fused", cfg),
                "fused_vs_separate_us": {
                    "fused": dom["avg_us"],
                    "quantize_act_plus_grouped_gemm": (kout["fp8q_quantize_act"]["avg_us"]
                                                       + kout["fp8q_grouped_gemm"]["avg_us"])}}
    elif args.workload in ("dense", "largek"):
        dom = kout["fp8q_gemm"]
        traffic = recorded_traffic("fp8q_gemm", cfg)
        roof = {"kernel": "fp8q_gemm", "bound": "mfma", "achieved": dom["TFLOP_s"],
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": dom["TFLOP_s"] / PEAK_FP8_TFLOPS,
                "traffic": traffic}
    else:
        dom = kout["fp8q_grouped_gemm"]
        dom["TFLOP_s"] = flops / (dom["avg_us"] * 1e-6) / 1e12
        dom["frac_fp8_peak"] = dom["TFLOP_s"] / PEAK_FP8_TFLOPS
        roof = {"kernel": "fp8q_grouped_gemm", "bound": "hbm", "achieved": dom["GB_s"],
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dom["GB_s"] / PEAK_HBM_GBS,
                "traffic": recorded_traffic("fp8q_grouped_gemm", cfg)}

    value = flops / (ms_per_step * 1e-3) / 1e12
    bf16 = args.workload == "bf16"
    rec = {"metric": METRIC_BF16 if bf16 else METRIC, "value": value, "unit": "TFLOP/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if bf16 else "fp8e4m3",
           "data": "synthetic (seeded; shapes and distributions of the workload table)",
           "config": cfg, "roofline": roof, "kernels": kout}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(base)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
