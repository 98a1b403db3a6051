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

Prints ONE JSON line (rank 0).  ``--gpus`` above 1 is refused: the benchmark
measures one GPU.
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
    p.add_argument("--mfma-scaled", action="store_true",
                   help="dense / largek: power-of-two scales, applied by the matrix core "
                        "(fp8q_gemm_mfma_scaled), timed beside fp8q_gemm on the same operands")
    p.add_argument("--precise", action="store_true",
                   help="the precise GEMM calls (fp8q_gemm_precise, fp8q_grouped_gemm_precise, "
                        "fp8q_gemm_rowscaled_precise) in place of the FP8-MFMA ones")
    p.add_argument("--sets", type=int, default=0, help="input sets rotated (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a streaming device copy of MIB MiB (3 times): the known-size "
                        "kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters")
    p.add_argument("--stream-ceiling", action="store_true",
                   help="only time the streaming probe (16 B read, 8 B written per lane: the "
                        "quantizers' 2:1 traffic) at the quantizers' sizes: their HBM ceiling")
    p.add_argument("--mix-probe", action="store_true",
                   help="only time the instruction-mix probe: MFMA streams with the GEMM main "
                        "loop's LDS fragment reads, promotion FMAs and FP8->FP16 widening")
    p.add_argument("--ring-probe", action="store_true",
                   help="only time the ring-streaming probe: the grouped GEMM's operand "
                        "pipeline alone (no MFMA) for its tile shapes and ring depths")
    return p.parse_args()


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "fine_grained_block_fp8q_amd", "libfp8q_probe.so")
    L = ctypes.CDLL(path)
    L.fp8q_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int, ctypes.c_void_p]
    L.fp8q_probe_stream.restype = ctypes.c_int
    return L


def _probe(L, torch, src, dst, nbytes, ratio):
    import ctypes
    st = L.fp8q_probe_stream(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                             nbytes, ratio,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError(f"fp8q_probe_stream failed: {st}")


def copy_probe(mib):
    import torch
    L = _probe_lib()
    n = mib * 1024 * 1024
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        _probe(L, torch, x, y, n, 1)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n, "launches": 3}))


def stream_ceiling(steps, rounds=10):
    """The quantizers against the streaming probe at the same bytes, in one
    process on the same buffers: for each activation shape, the probe (16 B
    read, 8 B written per lane: the quantizer's 2:1 traffic) reads the BF16
    input the quantizer reads and writes into its code buffer; each round
    times `steps` back-to-back launches of each between HIP events on the
    launch stream, over 4 rotating input sets (1 at >= 1 GiB), the two
    interleaved, which one goes first alternating between rounds; medians
    over `rounds` rounds.  GB/s counts read + written
    bytes (the quantizer's: its algorithmic 3.03125 B per element)."""
    import torch
    import fine_grained_block_fp8q_amd as fq
    L = _probe_lib()
    sizes = [("dense 4096x7168", 4096, 7168), ("decode 3980x7168", 3980, 7168),
             ("moe 32768x7168", 32768, 7168), ("largek 8192x65536", 8192, 65536),
             ("backward dY 4096x4096", 4096, 4096)]
    out = []
    for name, M, K in sizes:
        nin = 2 * M * K
        sets = 4 if nin < (1 << 30) else 1
        g = torch.Generator(device="cuda:0").manual_seed(M + K)
        xs = [torch.randn((M, K), generator=g, device="cuda:0").to(torch.bfloat16)
              for _ in range(sets)]
        qs = [torch.empty((M, K), dtype=torch.uint8, device="cuda:0") for _ in range(sets)]
        ss = [torch.empty((K // 128, M), dtype=torch.float32, device="cuda:0") for _ in range(sets)]
        quant = [fq.bind(fq.fp8q_quantize_act, xs[i], qs[i], ss[i]) for i in range(sets)]
        probe = [(lambda i=i: _probe(L, torch, xs[i], qs[i], nin, 2)) for i in range(sets)]
        times = {"probe": [], "quantizer": []}
        for r in range(rounds):
            order = (("probe", probe), ("quantizer", quant))
            for key, fns in (order if r % 2 == 0 else order[::-1]):
                fns[0]()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(steps):
                    fns[i % sets]()
                e1.record()
                torch.cuda.synchronize()
                times[key].append(e0.elapsed_time(e1) * 1e3 / steps)
        tp, tq = float(np.median(times["probe"])), float(np.median(times["quantizer"]))
        out.append({"case": name, "probe_us": tp, "probe_GB_s": 1.5 * nin / tp / 1e3,
                    "quantize_act_us": tq,
                    "quantize_act_GB_s": M * K * ACT_BYTES_PER_ELEM / tq / 1e3,
                    "quantize_act_frac_hbm": M * K * ACT_BYTES_PER_ELEM / tq / 1e3 / PEAK_HBM_GBS,
                    "quantize_act_over_probe_time": tq / tp})
        del xs, qs, ss, quant, probe
        torch.cuda.synchronize()
    print(json.dumps({"stream_ceiling": out, "steps": steps, "rounds": rounds,
                      "input_sets": "4 (1 at >= 1 GiB)"}))


MIX_KINDS = [  # (kind bits, what one iteration issues per wave)
    (0, "FP8: 4 MFMA 16x16x128 chained through C"),
    (1, "FP8: + 3 LDS reads (16 B) feeding the next operands"),
    (2, "FP8: MFMA from zero + 16 promotion FMAs"),
    (3, "FP8: + 3 LDS reads + 16 promotion FMAs (the fp8q_gemm mix)"),
    (16, "FP8 with E8M0 operand scales: 4 MFMA chained through C"),
    (19, "FP8 with E8M0 scales: + reads + promotion (the fp8q_gemm_mfma_scaled mix)"),
    (8, "FP16: 16 MFMA 16x16x32, 4 chained per block"),
    (9, "FP16: + 3 LDS reads"),
    (10, "FP16: + 16 promotion FMAs"),
    (11, "FP16: + 3 LDS reads + 16 promotion FMAs"),
    (13, "FP16: + 3 LDS reads widened by 24 FP8->FP16 conversions"),
    (15, "FP16: + reads + 24 conversions + 16 FMAs (the fp8q_gemm_precise mix)"),
]


def mix_probe(iters=20000, rounds=5):
    """The instruction-mix probe of libfp8q_probe.so (one workgroup of 8 waves
    per CU, two waves per SIMD): for each mix, the median over `rounds` of one
    launch's duration (HIP events) divided by `iters`, i.e. ns per iteration
    per wave; `mfma_share` = the time of the same mode's MFMA-only mix over
    this mix's time, the share of the matrix core's time that survives."""
    import ctypes
    import torch
    L = _probe_lib()
    L.fp8q_probe_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.fp8q_probe_mix.restype = ctypes.c_int
    L.fp8q_probe_cus.restype = ctypes.c_int
    cus = L.fp8q_probe_cus()
    if cus <= 0:
        raise RuntimeError("fp8q_probe_cus failed")
    out = torch.empty(cus * 512, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run(kind, n):
        st = L.fp8q_probe_mix(kind, n, ctypes.c_void_p(out.data_ptr()), stream)
        if st != 0:
            raise RuntimeError(f"fp8q_probe_mix({kind}) failed: {st}")

    ns = {}
    for r in range(rounds):
        for kind, _ in MIX_KINDS:
            run(kind, 100)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run(kind, iters)
            e1.record()
            torch.cuda.synchronize()
            ns.setdefault(kind, []).append(e0.elapsed_time(e1) * 1e6 / iters)
    rows = []
    for kind, what in MIX_KINDS:
        t = float(np.median(ns[kind]))
        t0 = float(np.median(ns[kind & 8]))   # the unscaled MFMA-only stream of the mode
        rows.append({"kind": kind, "mix": what, "ns_per_iter_per_wave": t, "mfma_share": t0 / t})
    print(json.dumps({"mix_probe": rows, "iters": iters, "rounds": rounds, "workgroups": cus,
                      "waves_per_simd": 2}))


RING_SHAPES = [  # (activation rows per tile, ring stages): the grouped GEMM's tiles
    (0, 2), (0, 3), (0, 4), (64, 3), (128, 3), (160, 3), (192, 2), (256, 2)]
RING_READ_SHAPES = [  # (activation rows, stages, LDS reads per wave and chunk)
    (0, 2, 24), (128, 3, 12), (128, 3, 24), (256, 2, 24)]
RING_SPLIT_SHAPES = [  # (activation rows, activation stages, weight stages): split rings
    (64, 2, 4), (128, 2, 3), (128, 2, 4), (128, 3, 3), (192, 2, 2), (192, 2, 3), (256, 2, 2),
    (256, 2, 3)]


def ring_probe(rounds=5):
    """The ring-streaming probe of libfp8q_probe.so: one workgroup per CU
    streams tiles of 256 weight rows of its own plus `ra` activation rows
    shared by the 16 tiles of an expert, K = 7168, through an LDS ring of
    `stages` stages, with no MFMA; then the split variant, whose activation
    rows and weight rows have rings of their own depths (`a_stages`,
    `w_stages`).  Regimes: 16 tiles per CU (7.5 GB of weights, the MoE
    batch's volume) and 2 tiles per CU (0.94 GB, the decode batch's), and an
    L2-resident one (all tiles read the same weight rows).  Median over
    `rounds` launches (HIP events); weight GB/s counts the weight bytes, total
    GB/s adds the activation bytes each tile reads.  Ends with the decode and
    MoE ceilings these rates give (ring_ceilings)."""
    import ctypes
    import torch
    L = _probe_lib()
    L.fp8q_probe_ring.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.fp8q_probe_ring.restype = ctypes.c_int
    L.fp8q_probe_ring_split.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    L.fp8q_probe_ring_split.restype = ctypes.c_int
    L.fp8q_probe_ring_reads.argtypes = L.fp8q_probe_ring_split.argtypes
    L.fp8q_probe_ring_reads.restype = ctypes.c_int
    L.fp8q_probe_cus.restype = ctypes.c_int
    cus = L.fp8q_probe_cus()
    K, per_expert = 7168, 16
    w = torch.empty((cus * 16 * 256, K), dtype=torch.uint8, device="cuda:0")
    a = torch.empty((256 * 256, K), dtype=torch.uint8, device="cuda:0")
    w.fill_(0x38)
    a.fill_(0x38)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rows = []
    # (act rows, act stages, stages, variant): variant 0 the kernel's ring, 1
    # split rings, or ("reads", n) the kernel's ring with n LDS reads per wave
    shapes = [(ra, s, s, 0) for ra, s in RING_SHAPES] + \
        [(ra, sa, sw, 1) for ra, sa, sw in RING_SPLIT_SHAPES] + \
        [(ra, s, s, ("reads", rd)) for ra, s, rd in RING_READ_SHAPES]
    # Regimes: weights from HBM at the MoE and decode volumes, and a check of
    # the CU side, where every tile reads the same 256 weight rows and one
    # expert's activation rows, so that after the first touch both hit in L2.
    regimes = [(16, "hbm", shapes), (2, "hbm", shapes),
               (16, "l2", [x for x in shapes if x[3] == 0 and x[0] in (0, 128, 256)])]
    for tiles, src, rshapes in regimes:
        w_rows = cus * tiles * 256 if src == "hbm" else 256
        for ra, a_st, stages, split in rshapes:
            a_rows = (256 * ra if src == "hbm" else ra) if ra else 0

            def run():
                if isinstance(split, tuple):
                    st = L.fp8q_probe_ring_reads(ctypes.c_void_p(w.data_ptr()), w_rows,
                                                 ctypes.c_void_p(a.data_ptr()), a_rows, K, ra,
                                                 stages, split[1], tiles, per_expert, stream)
                elif split:
                    st = L.fp8q_probe_ring_split(ctypes.c_void_p(w.data_ptr()), w_rows,
                                                 ctypes.c_void_p(a.data_ptr()), a_rows, K, ra,
                                                 a_st, stages, tiles, per_expert, stream)
                else:
                    st = L.fp8q_probe_ring(ctypes.c_void_p(w.data_ptr()), w_rows,
                                           ctypes.c_void_p(a.data_ptr()), a_rows, K, ra, stages,
                                           tiles, per_expert, stream)
                if st != 0:
                    raise RuntimeError(f"ring probe ({ra}, {a_st}, {stages}, split={split}) "
                                       f"failed: {st}")

            run()
            ts = []
            for _ in range(rounds):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                run()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            us = float(np.median(ts))
            wb = cus * tiles * 256 * K
            ab = cus * tiles * ra * K
            rows.append({"tiles_per_cu": tiles, "weights": src, "act_rows": ra,
                         "split": split == 1,
                         "lds_reads": split[1] if isinstance(split, tuple) else 0,
                         "act_stages": a_st, "stages": stages, "us": us,
                         "weight_GB_s": wb / us / 1e3, "total_GB_s": (wb + ab) / us / 1e3})
            print(json.dumps(rows[-1]), flush=True)
    print(json.dumps({"ring_probe": rows, "K": K, "weight_rows_per_tile": 256,
                      "tiles_per_expert": per_expert, "workgroups": cus, "rounds": rounds,
                      "ceilings": ring_ceilings(rows)}))


# The grouped GEMM's row buckets (tile rows <= bucket) with their ring depths.
GROUPED_BUCKETS = [(64, 3), (128, 3), (160, 3), (192, 2), (256, 2)]


def ring_ceilings(rows):
    """Streaming ceiling of the decode and MoE workloads from the ring probe's
    rates: every m-tile of an expert (at most 256 rows) runs N/256 tiles in its
    row bucket's ring, each streaming 256 x K weight bytes at that bucket's
    measured weight rate (2 tiles per CU for decode, 16 for MoE, as the two
    batches load the chip); the tiles' times add up.  The output writes are
    left out, so the ceiling is optimistic.  GB/s = algorithmic bytes / time."""
    import workloads
    out = {}
    for name, tiles_per_cu in (("decode", 2), ("moe", 16)):
        c = workloads.WORKLOADS[name]
        N, K = c["N"], c["K"]
        if name == "moe":
            counts, _, _ = workloads.moe_routing(c["tokens"], c["experts"], c["topk"], c["seed"])
            ob = 4
        else:
            counts, _ = workloads.decode_counts(c["experts"], c["m_lo"], c["m_hi"], c["seed"])
            ob = 2
        rate = {ra: r["weight_GB_s"] for r in rows for ra, st in GROUPED_BUCKETS
                if not r["split"] and r["tiles_per_cu"] == tiles_per_cu
                and r.get("weights", "hbm") == "hbm" and not r.get("lds_reads", 0)
                and r["act_rows"] == ra and r["stages"] == st}
        t_us, per_bucket = 0.0, {}
        for m in counts:
            m = int(m)
            while m > 0:
                live = min(m, 256)
                b = next(ra for ra, _ in GROUPED_BUCKETS if live <= ra)
                per_bucket[b] = per_bucket.get(b, 0) + 1
                t_us += (N // 256) * 256 * K / (rate[b] * 1e3)
                m -= live
        G, Mt = len(counts), int(counts.sum())
        gbytes = G * N * K * (1 + 4 / 16384) + Mt * K * (1 + 4 / 128) + Mt * N * ob
        out[name] = {"us": t_us, "GB_s": gbytes / t_us / 1e3,
                     "frac_hbm": gbytes / t_us / 1e3 / PEAK_HBM_GBS,
                     "m_tiles_per_bucket": {str(k): v for k, v in sorted(per_bucket.items())}}
    return out


def gemm_bytes(M, N, K, out_bytes):
    return M * K * (1 + 4 / 128) + N * K * (1 + 4 / 16384) + M * N * out_bytes


# --------------------------------------------------------------------- setup
def setup_dense(fq, torch, name, sets, fused=False, precise=False, mfma_scaled=False):
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

    # every call validated once by the binding, then repeated without the
    # per-call host checks (fq.bind): the launch loops below must not be
    # host-bound for the shorter kernels
    calls = {n: [] for n in ("fp8q_quantize_act", "fp8q_quantize_weight", "fp8q_gemm_fused",
                             "fp8q_gemm_precise", "fp8q_gemm_mfma_scaled", "fp8q_gemm")}
    mode = "pow2" if mfma_scaled else "f32"
    for A, W, aq, as_, wq, ws, C in bufs:
        calls["fp8q_quantize_act"].append(fq.bind(fq.fp8q_quantize_act, A, aq, as_, mode))
        calls["fp8q_quantize_weight"].append(fq.bind(fq.fp8q_quantize_weight, W, wq, ws, mode))
        calls["fp8q_gemm_mfma_scaled"].append(
            fq.bind(fq.fp8q_gemm_mfma_scaled, aq, as_, wq, ws, C))
        calls["fp8q_gemm_fused"].append(fq.bind(fq.fp8q_gemm_fused, A, wq, ws, C))
        calls["fp8q_gemm_precise"].append(fq.bind(fq.fp8q_gemm_precise, aq, as_, wq, ws, C))
        calls["fp8q_gemm"].append(fq.bind(fq.fp8q_gemm, aq, as_, wq, ws, C))

    def launch(name, i):
        calls[name][i % sets]()

    gname = ("fp8q_gemm_precise" if precise else
             "fp8q_gemm_mfma_scaled" if mfma_scaled else "fp8q_gemm")
    order = (["fp8q_quantize_weight", "fp8q_gemm_fused"] if fused else
             ["fp8q_quantize_act", "fp8q_quantize_weight", gname])

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
    if precise:
        kernels.insert(0, ("fp8q_gemm_precise", "mfma_wide16", 2.0 * M * N * K, "flop"))
    if mfma_scaled:
        kernels.insert(0, ("fp8q_gemm_mfma_scaled", "mfma", 2.0 * M * N * K, "flop"))
    flops = 2.0 * M * N * K
    tag = (name + ("_fused" if fused else "") + ("_precise" if precise else "")
           + ("_mfma_scaled" if mfma_scaled else ""))
    how = "quantized inside the GEMM" if fused else "1x128 act quant"
    if precise:
        how += "; precise GEMM (codes widened to FP16, FP16 MFMA)"
    if mfma_scaled:
        how += "; power-of-two scales applied by the matrix core (E8M0)"
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
    # Same-chip context for the FP8 GEMMs: hipBLASLt's FP8 GEMM through
    # torch._scaled_mm with one scale per tensor (no per-block promotion), on
    # the codes of the first input set, BF16 out.
    A, W, Wt, aq, as_, wq, ws, C, Cb = bufs[0]
    one = torch.ones((), dtype=torch.float32, device=dev)
    a8 = aq.view(torch.float8_e4m3fn)
    w8t = wq.view(torch.float8_e4m3fn).t()  # [K][N] column-major view, as _scaled_mm wants
    try:
        torch._scaled_mm(a8, w8t, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        have_scaled_mm = True
    except Exception as e:  # not every build supports it
        have_scaled_mm = False
        print(f"torch._scaled_mm unavailable: {e}", file=sys.stderr)

    calls = {n: [] for n in ("fp8q_gemm_bf16", "fp8q_gemm", "fp8q_gemm_precise")}
    for A, W, Wt, aq, as_, wq, ws, C, Cb in bufs:
        calls["fp8q_gemm_bf16"].append(fq.bind(fq.fp8q_gemm_bf16, A, W, C))
        calls["fp8q_gemm"].append(fq.bind(fq.fp8q_gemm, aq, as_, wq, ws, C))
        calls["fp8q_gemm_precise"].append(fq.bind(fq.fp8q_gemm_precise, aq, as_, wq, ws, C))

    def launch(name, i):
        A, W, Wt, aq, as_, wq, ws, C, Cb = bufs[i % sets]
        if name in calls:
            calls[name][i % sets]()
        elif name == "torch_scaled_mm_fp8_per_tensor_hipblaslt":
            torch._scaled_mm(a8, w8t, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        else:  # hipBLASLt through torch, BF16 out
            torch.matmul(A, Wt, out=Cb)

    def step(i):
        launch("fp8q_gemm_bf16", i)

    flops = 2.0 * M * N * K
    kernels = [
        ("fp8q_gemm_bf16", "mfma_bf16", flops, "flop"),
        ("torch_matmul_bf16_hipblaslt", "mfma_bf16", flops, "flop"),
        ("fp8q_gemm", "mfma", flops, "flop"),
        ("fp8q_gemm_precise", "mfma_wide16", flops, "flop"),
    ]
    if have_scaled_mm:
        kernels.append(("torch_scaled_mm_fp8_per_tensor_hipblaslt", "mfma", flops, "flop"))
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

    calls = {}
    for b in bufs:
        for name, fn, a in (
                ("fp8q_quantize_act", fq.fp8q_quantize_act, (b["dY"], b["qd"], b["sd"])),
                ("fp8q_quantize_weight_t", fq.fp8q_quantize_weight_t, (b["W"], b["qwt"], b["swt"])),
                ("fp8q_gemm", fq.fp8q_gemm, (b["qd"], b["sd"], b["qwt"], b["swt"], b["dX"])),
                ("fp8q_quantize_act_t:dY", fq.fp8q_quantize_act_t, (b["dY"], b["qdt"], b["sdt"])),
                ("fp8q_quantize_act_t:X", fq.fp8q_quantize_act_t, (b["X"], b["qxt"], b["sxt"])),
                ("fp8q_gemm_rowscaled", fq.fp8q_gemm_rowscaled,
                 (b["qdt"], b["sdt"], b["qxt"], b["sxt"], b["dW"]))):
            calls.setdefault(name, []).append(fq.bind(fn, *a))

    def launch(name, i):
        calls[name][i % sets]()

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


def setup_grouped(fq, torch, name, sets, fused=False, precise=False):
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

    calls = {n: [] for n in ("fp8q_quantize_act", "fp8q_grouped_gemm_fused",
                             "fp8q_grouped_gemm_precise", "fp8q_grouped_gemm")}
    for A, aq, as_, C in bufs:
        calls["fp8q_quantize_act"].append(fq.bind(fq.fp8q_quantize_act, A, aq, as_))
        calls["fp8q_grouped_gemm_fused"].append(
            fq.bind(fq.fp8q_grouped_gemm_fused, A, d_off, wq, ws, C))
        calls["fp8q_grouped_gemm_precise"].append(
            fq.bind(fq.fp8q_grouped_gemm_precise, aq, as_, d_off, wq, ws, C))
        calls["fp8q_grouped_gemm"].append(fq.bind(fq.fp8q_grouped_gemm, aq, as_, d_off, wq, ws, C))

    def launch(name, i):
        calls[name][i % sets]()

    gname = "fp8q_grouped_gemm_precise" if precise else "fp8q_grouped_gemm"

    def step(i):
        if fused:
            launch("fp8q_grouped_gemm_fused", i)
        else:
            launch("fp8q_quantize_act", i)
            launch(gname, i)

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
    if precise:
        kernels.insert(0, ("fp8q_grouped_gemm_precise", "hbm", gbytes, "B"))
    tag = name + ("_fused" if fused else "") + ("_precise" if precise else "")
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


def recorded(kind, kernel, cfg):
    """The fields of the committed `kind` record line ("traffic-record" or
    "clock-record") of profiles/*.md for this kernel and workload, or None if
    there is none or the GEMM code changed since it was measured."""
    import glob
    digest = kernel_source_digest()
    workload = cfg["workload"].split(":")[0]
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith(kind + ":"):
                continue
            rec = dict(kv.split("=", 1) for kv in line.split(":", 1)[1].split())
            if (rec.get("kernel") == kernel and rec.get("workload") == workload
                    and rec.get("source_sha256") == digest):
                return rec
    return None


def recorded_ceiling(kernel, cfg):
    """Algorithmic GB/s of the workload's tile shapes streamed without
    arithmetic (the `ceiling-record` lines of profiles/*.md, written from
    bench.py --ring-probe), or None."""
    import glob
    workload = cfg["workload"].split(":")[0]
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if line.startswith("ceiling-record:"):
                rec = dict(kv.split("=", 1) for kv in line.split(":", 1)[1].split())
                if rec.get("kernel") == kernel and rec.get("workload") == workload:
                    return float(rec["GB_s"])
    return None


def recorded_traffic(kernel, cfg):
    """HBM-side bytes per launch from the committed rocprofv3 --pmc summary
    (FETCH_SIZE and WRITE_SIZE, calibrated on a copy of known size), or None
    if there is none for this kernel and workload or the kernel changed."""
    rec = recorded("traffic-record", kernel, cfg)
    return float(rec["bytes_per_launch"]) if rec else None


# ------------------------------------------------------------ shader clock
PEAK_CLOCK_MHZ = 2400.0   # the clock the published MFMA peaks assume


# --------------------------------------------------------------- cpu baseline
def _cpu_model():
    """The host CPU's model name as lscpu reports it (else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_sample(name):
    """(run, flops, what, full_flops): one run of the oracle on a bounded
    sample of the workload, its flops, a description, the whole workload's
    flops (the rate is extrapolated to it when they differ)."""
    import workloads
    from oracle import gemm as ogemm, quant as oquant
    if name == "backward":
        c = workloads.WORKLOADS["dense"]
        M, N, K = c["M"], c["N"], c["K"]
        rows = 256
        X, _ = workloads.dense_inputs("dense", rows_w=np.arange(128))
        dY = workloads.bf16_bits(
            (np.random.default_rng(c["seed"] + 7).standard_normal((M, N)) * 1e-2).astype(np.float32))

        def run():
            qdt, sdt = oquant.quantize_act_t(dY)
            qxt, sxt = oquant.quantize_act_t(X)
            ogemm.gemm_rowscaled(qdt[:rows], sdt[:, :rows], qxt, sxt)
        return (run, 2.0 * rows * K * M,
                f"Wgrad rows 0..{rows - 1} of dW: oracle quantize_act_t of dY ({M}x{N}) and X "
                f"({M}x{K}) + exact row-scaled GEMM {rows}x{K}x{M}", 2.0 * 2 * M * N * K)
    if name == "bf16":
        c = workloads.WORKLOADS["dense"]
        M, N, K = 1024, 1024, c["K"]
        A, W = workloads.dense_inputs("dense", rows_a=np.arange(M), rows_w=np.arange(N))
        return (lambda: ogemm.gemm_bf16(A, W), 2.0 * M * N * K,
                f"rows 0..{M - 1} of A and 0..{N - 1} of W: oracle gemm_bf16 (float64 matmul "
                f"of the BF16 values) {M}x{N}x{K}", 2.0 * c["M"] * c["N"] * K)
    c = workloads.WORKLOADS[name]
    if name in ("dense", "largek"):
        M, N = (2048, 2048) if name == "dense" else (64, 512)
        K = c["K"]
        A, W = workloads.dense_inputs(name, rows_a=np.arange(M), rows_w=np.arange(N))
        what = f"rows 0..{M - 1} of A and 0..{N - 1} of W"
        full = 2.0 * c["M"] * c["N"] * K
    else:
        M, N, K = 256, c["N"], c["K"]
        outl = workloads.outlier_channels(K, c["seed"], c["outlier_frac"], c["outlier_count"])
        A = workloads.act_rows(np.arange(M), K, c["seed"], c["act_std"], outl, c["outlier_mult"])
        W = workloads.weight_rows(np.arange(N), K, c["seed"], c["w_std"])
        what = f"{M} activation rows x one expert's {N}x{K} weight"
        if name == "moe":
            full = 2.0 * c["tokens"] * c["topk"] * N * K
        else:
            counts, _ = workloads.decode_counts(c["experts"], c["m_lo"], c["m_hi"], c["seed"])
            full = 2.0 * float(counts.sum()) * N * K

    def run():
        qa, sa = oquant.quantize_act(A)
        qw, sw = oquant.quantize_weight(W)
        ogemm.gemm(qa, sa, qw, sw)
    return (run, 2.0 * M * N * K,
            f"{what}: oracle quantize_act({M}x{K}) + quantize_weight({N}x{K}) + exact float64 "
            f"per-chunk GEMM {M}x{N}x{K}", full)


def cpu_baseline(name):
    """The oracle, untuned, on the host: a bounded sample of the workload run
    3 times with every BLAS thread the process may use and 3 times on one
    thread; wall clock of each run (input generation excluded), median
    reported.  value = sample flops / median wall (TFLOP/s), extrapolated to
    the whole workload when the sample is a slice."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threadpool_limits = None
        blas = os.cpu_count() or 1
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    run, flops, what, full = _cpu_sample(name)

    def median_wall(reps=3):
        walls = []
        for _ in range(reps):
            t0 = time.perf_counter()
            run()
            walls.append(time.perf_counter() - t0)
        return float(np.median(walls)), walls

    wall_all, walls_all = median_wall()
    wall_one, walls_one = None, []
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            wall_one, walls_one = median_wall()
    sliced = abs(full - flops) > 1e-6 * full
    rec = {"value": flops / wall_all / 1e12, "unit": "TFLOP/s", "cores": int(blas),
           "kind": "oracle",
           "sample": f"{what}; median of 3 runs {', '.join(f'{w:.2f}' for w in walls_all)} s; "
                     f"value = sample flops / median wall"
                     + ("; extrapolated: the rate is taken to hold for the whole workload"
                        if sliced else "; the whole workload"),
           "value_1core": (flops / wall_one / 1e12) if wall_one else None,
           "walls_1core_s": walls_one,
           "extrapolated": bool(sliced),
           "workload_time_s": full / (flops / wall_all) if sliced else wall_all,
           "cpu_model": _cpu_model(), "usable_cpus": int(usable or 1),
           "blas_threads": int(blas)}
    return rec


# ----------------------------------------------------------------------- main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.mfma_scaled and (args.precise or args.workload not in ("dense", "largek")):
        print(json.dumps({"error": "--mfma-scaled applies to the dense and largek workloads only"}))
        sys.exit(2)
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.stream_ceiling:
        stream_ceiling(args.steps)
        return
    if args.mix_probe:
        mix_probe()
        return
    if args.ring_probe:
        ring_probe()
        return
    import torch
    import fine_grained_block_fp8q_amd as fq

    sets = args.sets or (4 if args.workload in ("dense", "bf16", "dense_fused") else
                         2 if args.workload in ("decode", "backward", "decode_fused") else 1)
    base = args.workload.replace("_fused", "")
    fused = base != args.workload
    if base in ("dense", "largek"):
        step, launch, kernels, flops, cfg = setup_dense(fq, torch, base, sets, fused, args.precise,
                                                        args.mfma_scaled)
    elif args.workload == "bf16":
        step, launch, kernels, flops, cfg = setup_bf16(fq, torch, sets)
    elif args.workload == "backward":
        step, launch, kernels, flops, cfg = setup_backward(fq, torch, sets)
    else:
        step, launch, kernels, flops, cfg = setup_grouped(fq, torch, base, sets, fused,
                                                          args.precise)
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
    # Before each kernel's loops, one read-only pass over 512 MiB evicts what
    # the previous loops left in the 256 MB last-level cache: the dirty lines
    # of the timed steps' GEMM outputs would otherwise be written back during
    # the next kernel's timing and charged to it.
    settle_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    kout = {}
    for kname, bound, work, unit in kernels:
        settle_buf.max()
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
                              else ("frac_fp16_peak", PEAK_BF16_TFLOPS) if bound == "mfma_wide16"
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
    elif args.mfma_scaled and args.workload in ("dense", "largek"):
        dom = kout["fp8q_gemm_mfma_scaled"]
        roof = {"kernel": "fp8q_gemm_mfma_scaled", "bound": "mfma", "achieved": dom["TFLOP_s"],
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": dom["TFLOP_s"] / PEAK_FP8_TFLOPS,
                "traffic": recorded_traffic("fp8q_gemm_mfma_scaled", cfg),
                "vs_fp8q_gemm_same_operands_us": {
                    "mfma_scaled": dom["avg_us"], "fp8q_gemm": kout["fp8q_gemm"]["avg_us"]}}
    elif args.precise and args.workload in ("dense", "largek"):
        dom = kout["fp8q_gemm_precise"]
        roof = {"kernel": "fp8q_gemm_precise", "bound": "mfma", "achieved": dom["TFLOP_s"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": dom["TFLOP_s"] / PEAK_BF16_TFLOPS,
                "frac_of_fp8_peak": dom["TFLOP_s"] / PEAK_FP8_TFLOPS,
                "peak_note": "FP16 MFMA dense peak (the instruction the precise mode runs); "
                             "frac_of_fp8_peak against the FP8 dense peak",
                "traffic": recorded_traffic("fp8q_gemm_precise", cfg)}
    elif args.precise:
        dom = kout["fp8q_grouped_gemm_precise"]
        dom["TFLOP_s"] = flops / (dom["avg_us"] * 1e-6) / 1e12
        dom["frac_fp8_peak"] = dom["TFLOP_s"] / PEAK_FP8_TFLOPS
        dom["frac_fp16_peak"] = dom["TFLOP_s"] / PEAK_BF16_TFLOPS
        roof = {"kernel": "fp8q_grouped_gemm_precise", "bound": "hbm", "achieved": dom["GB_s"],
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dom["GB_s"] / PEAK_HBM_GBS,
                "traffic": recorded_traffic("fp8q_grouped_gemm_precise", cfg)}
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

    # Clock-normalised figures: the shader clock the dominant kernel holds,
    # from its committed rocprofv3 counter record (GRBM_GUI_ACTIVE per XCD over
    # the dispatch's duration; reported while the GEMM code is unchanged),
    # and its per-launch median beside the back-to-back average the fraction
    # is based on.
    clk = recorded("clock-record", roof["kernel"], cfg)
    if clk:
        roof["sclk_MHz_profiled"] = float(clk["sclk_MHz"])
        roof["mfma_busy_profiled"] = float(clk["mfma_busy"])
        if roof["unit"] == "TFLOP/s":
            roof["peak_at_sclk"] = roof["peak"] * roof["sclk_MHz_profiled"] / PEAK_CLOCK_MHZ
            roof["frac_at_sclk"] = roof["achieved"] / roof["peak_at_sclk"]
    # The streaming ceiling of an HBM-bound kernel's tile shapes, from the
    # committed ring-probe summary (the probe, not the GEMM, measures it).
    if roof["unit"] == "GB/s":
        ceil = recorded_ceiling(roof["kernel"], cfg)
        if ceil:
            roof["stream_ceiling_GB_s"] = ceil
            roof["frac_of_stream_ceiling"] = roof["achieved"] / ceil
    med = dom.get("median_us")
    if med:
        roof["median_launch_us"] = med
        roof["frac_by_median_launch"] = roof["frac"] * dom["avg_us"] / med

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
