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
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
ACT_BYTES_PER_ELEM = 2 + 1 + 4 / 128          # BF16 in, E4M3 out, one FP32 scale per 128
WEIGHT_BYTES_PER_ELEM = 2 + 1 + 4 / 16384     # one FP32 scale per 128x128 block


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dense", choices=["dense", "moe", "decode", "largek"])
    p.add_argument("--sets", type=int, default=0, help="input sets rotated (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def gemm_bytes(M, N, K, out_bytes):
    return M * K * (1 + 4 / 128) + N * K * (1 + 4 / 16384) + M * N * out_bytes


# --------------------------------------------------------------------- setup
def setup_dense(fq, torch, name, sets):
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

    def step(i, ev):
        A, W, aq, as_, wq, ws, C = bufs[i % sets]
        ev[0].record()
        fq.fp8q_quantize_act(A, aq, as_)
        ev[1].record()
        fq.fp8q_quantize_weight(W, wq, ws)
        ev[2].record()
        fq.fp8q_gemm(aq, as_, wq, ws, C)
        ev[3].record()

    kernels = [
        ("fp8q_quantize_act", "hbm", M * K * ACT_BYTES_PER_ELEM, "B"),
        ("fp8q_quantize_weight", "hbm", N * K * WEIGHT_BYTES_PER_ELEM, "B"),
        ("fp8q_gemm", "mfma", 2.0 * M * N * K, "flop"),
    ]
    flops = 2.0 * M * N * K
    cfg = {"workload": f"{name}: A {M}x{K} bf16 (1x128 act quant), W {N}x{K} bf16 "
                       f"(128x128 block quant), C = A W^T fp32",
           "M": M, "N": N, "K": K, "out": "f32", "input_sets": sets}
    return step, kernels, flops, cfg, 2 + 1 + 1, (M, N, K)


def setup_grouped(fq, torch, name, sets):
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

    def step(i, ev):
        A, aq, as_, C = bufs[i % sets]
        ev[0].record()
        fq.fp8q_quantize_act(A, aq, as_)
        ev[1].record()
        ev[2].record()
        fq.fp8q_grouped_gemm(aq, as_, d_off, wq, ws, C)
        ev[3].record()

    ob = 2 if out_dtype == torch.bfloat16 else 4
    flops = 2.0 * Mt * N * K
    gbytes = G * N * K * (1 + 4 / 16384) + Mt * K * (1 + 4 / 128) + Mt * N * ob
    kernels = [
        ("fp8q_quantize_act", "hbm", Mt * K * ACT_BYTES_PER_ELEM, "B"),
        ("fp8q_grouped_gemm", "hbm", gbytes, "B"),
        ("fp8q_grouped_gemm:flops", "mfma", flops, "flop"),
    ]
    cfg = {"workload": f"{name}: {G} experts, rows {Mt} (M_e {int(counts.min())}..{int(counts.max())}), "
                       f"N {N}, K {K}, 1x128 act quant + grouped GEMM, weights pre-quantized 128x128",
           "experts": G, "rows": Mt, "N": N, "K": K, "out": "bf16" if ob == 2 else "f32",
           "input_sets": sets}
    return step, kernels, flops, cfg, None, (Mt, N, K)


# --------------------------------------------------------------- cpu baseline
def cpu_baseline(name):
    """The oracle, untuned, on a bounded sample of the workload (host cores)."""
    import workloads
    from oracle import gemm as ogemm, quant as oquant
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    c = workloads.WORKLOADS["dense" if name not in workloads.WORKLOADS else name]
    if name in ("moe", "decode"):
        M, N, K = 64, c["N"], c["K"]
        rows_w = np.arange(N)
    else:
        M, N, K = 32, min(c["N"], 4096), min(c["K"], 7168)
        rows_w = np.arange(N)
    if "M" in c:
        A, W = workloads.dense_inputs(name, rows_a=np.arange(M), rows_w=rows_w)
        A, W = A[:, :K], W[:, :K]
    else:
        A = workloads.act_rows(np.arange(M), K, c["seed"])
        W = workloads.weight_rows(rows_w, K, c["seed"], c["w_std"])
    t0 = time.perf_counter()
    qa, sa = oquant.quantize_act(A)
    qw, sw = oquant.quantize_weight(W)
    ogemm.gemm(qa, sa, qw, sw)
    dt = time.perf_counter() - t0
    flops = 2.0 * M * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle quantize_act({M}x{K}) + quantize_weight({N}x{K}) + exact float64 "
                      f"per-chunk GEMM {M}x{N}x{K}; {dt:.1f} s wall; value = 2*M*N*K / wall"}


# ----------------------------------------------------------------------- main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import fine_grained_block_fp8q_amd as fq

    sets = args.sets or (4 if args.workload in ("dense",) else 2 if args.workload == "decode" else 1)
    if args.workload in ("dense", "largek"):
        step, kernels, flops, cfg, _, shape = setup_dense(fq, torch, args.workload, sets)
    else:
        step, kernels, flops, cfg, _, shape = setup_grouped(fq, torch, args.workload, sets)
    torch.cuda.synchronize()

    nev = 4
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    for i in range(args.warmup):
        step(i, mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(nev - 1)]
                    for i in range(args.steps)])  # ms
    span = np.array([evs[i][0].elapsed_time(evs[i][nev - 1]) for i in range(args.steps)])
    ms_per_step = wall * 1e3 / args.steps

    ktimes = {}
    if args.workload in ("dense", "largek"):
        ktimes = {"fp8q_quantize_act": seg[:, 0], "fp8q_quantize_weight": seg[:, 1],
                  "fp8q_gemm": seg[:, 2]}
    else:
        ktimes = {"fp8q_quantize_act": seg[:, 0], "fp8q_grouped_gemm": seg[:, 2],
                  "fp8q_grouped_gemm:flops": seg[:, 2]}
    kout = {}
    for kname, bound, work, unit in kernels:
        avg_ms = float(np.mean(ktimes[kname]))
        if unit == "B":
            ach = work / (avg_ms * 1e-3) / 1e9
            kout[kname] = {"avg_us": avg_ms * 1e3, "median_us": float(np.median(ktimes[kname])) * 1e3,
                           "GB_s": ach, "frac_hbm": ach / PEAK_HBM_GBS, "bytes": work}
        else:
            ach = work / (avg_ms * 1e-3) / 1e12
            kout[kname] = {"avg_us": avg_ms * 1e3, "median_us": float(np.median(ktimes[kname])) * 1e3,
                           "TFLOP_s": ach, "frac_fp8_peak": ach / PEAK_FP8_TFLOPS, "flops": work}

    if args.workload in ("dense", "largek"):
        dom = kout["fp8q_gemm"]
        roof = {"kernel": "fp8q_gemm", "bound": "mfma", "achieved": dom["TFLOP_s"],
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": dom["TFLOP_s"] / PEAK_FP8_TFLOPS,
                "traffic": None}
    else:
        dom = kout["fp8q_grouped_gemm"]
        roof = {"kernel": "fp8q_grouped_gemm", "bound": "hbm", "achieved": dom["GB_s"],
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dom["GB_s"] / PEAK_HBM_GBS,
                "traffic": None}

    value = flops / (ms_per_step * 1e-3) / 1e12
    rec = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
           "data": "synthetic (seeded; shapes and distributions of the workload table)",
           "config": cfg, "roofline": roof, "kernels": kout,
           "event_ms_per_step": float(np.mean(span))}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
