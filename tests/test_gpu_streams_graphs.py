"""The entry points under concurrency and HIP graph capture, through the C ABI:

1. Calls on two streams at once (a dense GEMM with its quantizers on one, a
   grouped GEMM on the other) give bit for bit the outputs of the same calls
   made one after the other: the library keeps no state between calls.
2. A whole quantize + quantize + GEMM step captured into a HIP graph (the
   calls take torch's current stream, the capture stream) replays to the
   eager outputs, bit for bit, on three different inputs copied into the
   graph's input buffers between replays, with eager work and
   synchronizations in between.  None of the kernels needs a memset.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import DEV, fq, to_dev_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view({4: torch.int32, 2: torch.int16, 1: torch.uint8}[t.element_size()])


def _inputs(seed, M=512, N=768, K=1024):
    rng = np.random.default_rng(seed)
    A = workloads.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = workloads.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    return to_dev_bf16(A), to_dev_bf16(W)


def test_two_streams_match_serial():
    f = fq()
    a, w = _inputs(1)
    G, N, K = 6, 512, 1024
    rng = np.random.default_rng(2)
    off_h = np.concatenate([[0], np.cumsum(rng.integers(0, 200, size=G))]).astype(np.int32)
    Mg = int(off_h[-1])
    ag = to_dev_bf16(workloads.bf16_bits(rng.standard_normal((Mg, K)).astype(np.float32)))
    wg = to_dev_bf16(workloads.bf16_bits((rng.standard_normal((G * N, K)) * 0.02).astype(np.float32)))
    off = torch.from_numpy(off_h).to(DEV)
    gq, gs = f.quantize_act(ag)
    gwq, gws = f.quantize_weight(wg)
    gwq, gws = gwq.view(G, N, K), gws.view(G, N // 128, K // 128)

    def dense():
        aq, as_ = f.quantize_act(a)
        wq, ws = f.quantize_weight(w)
        return [aq, as_, wq, ws, f.gemm(aq, as_, wq, ws), f.gemm(aq, as_, wq, ws, precise=True)]

    def grouped():
        return [f.grouped_gemm(gq, gs, off, gwq, gws),
                f.grouped_gemm(gq, gs, off, gwq, gws, precise=True)]

    ref = dense() + grouped()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            out1 = dense()
        with torch.cuda.stream(s2):
            out2 = grouped()
        torch.cuda.synchronize()
        for r, o in zip(ref, out1 + out2):
            assert torch.equal(_bits(r), _bits(o)), "a concurrent call differs from the serial one"


def test_graph_capture_replays_the_eager_step():
    f = fq()
    a, w = _inputs(3)
    M, K = a.shape
    N = w.shape[0]
    aq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    as_ = torch.empty((K // 128, M), dtype=torch.float32, device=DEV)
    wq = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=DEV)
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    cp = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def step():
        f.fp8q_quantize_act(a, aq, as_)
        f.fp8q_quantize_weight(w, wq, ws)
        f.fp8q_gemm(aq, as_, wq, ws, c)
        f.fp8q_gemm_precise(aq, as_, wq, ws, cp)

    step()                      # warm: the library's one-time device check runs eagerly
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for seed in (4, 5, 6):
        na, nw = _inputs(seed)
        a.copy_(na)
        w.copy_(nw)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (aq, as_, wq, ws, c, cp)]
        step()                  # the same step, eagerly
        torch.cuda.synchronize()
        for x, y in zip(got, (aq, as_, wq, ws, c, cp)):
            assert torch.equal(_bits(x), _bits(y)), f"graph replay differs from eager (seed {seed})"
