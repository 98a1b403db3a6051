"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the method's arithmetic (no max-abs, scale, cast or
GEMM): only random matrices rounded to BF16, outlier channels, MoE routing
counts and the workload table.  Both the CPU oracle and the HIP path consume
its outputs; neither is imported here.

Row-seeded generation: row r of a matrix drawn with seed s comes from
``numpy.random.default_rng([s, tag, r])`` (PCG64), so any row can be
regenerated on its own (the oracle checks sampled rows of large shapes).
"""

import numpy as np

# Workload table: the five shapes the method is exercised on.  Activations are
# K-contiguous [M][K]; weights are [N][K] (gate+up projection of a 2048-wide
# expert stacked: N = 2 x 2048).
WORKLOADS = {
    "tiny": dict(M=128, N=256, K=512, seed=1001, act_std=1.0,
                 outlier_frac=None, outlier_count=2, outlier_mult=50.0,
                 w_std=0.02, out="f32"),
    "dense": dict(M=4096, N=4096, K=7168, seed=1002, act_std=1.0,
                  outlier_frac=0.01, outlier_count=None, outlier_mult=30.0,
                  w_std=0.02, out="f32"),
    "moe": dict(tokens=4096, experts=256, topk=8, N=4096, K=7168, seed=1003,
                act_std=1.0, outlier_frac=0.01, outlier_count=None,
                outlier_mult=30.0, w_std=0.02, out="f32"),
    "decode": dict(experts=32, m_lo=16, m_hi=256, N=4096, K=7168, seed=1004,
                   act_std=1.0, outlier_frac=0.01, outlier_count=None,
                   outlier_mult=30.0, w_std=0.02, out="bf16"),
    "largek": dict(M=8192, N=8192, K=65536, seed=1005, act_std=1.0,
                   outlier_frac=None, outlier_count=0, outlier_mult=1.0,
                   w_std=1.0, out="f32"),
}

_TAG_ACT, _TAG_W, _TAG_OUTLIER, _TAG_ROUTE, _TAG_COUNTS = 1, 2, 3, 4, 5


def bf16_bits(x):
    """float32 array -> BF16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def outlier_channels(K, seed, frac=None, count=None):
    """Sorted K-column indices chosen without replacement (same for every row)."""
    n = int(round(frac * K)) if frac is not None else int(count or 0)
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([seed, _TAG_OUTLIER])
    return np.sort(rng.choice(K, size=n, replace=False))


def act_rows(rows, K, seed, std=1.0, outliers=None, mult=1.0):
    """BF16 bits of the given activation rows: N(0, std^2), outlier columns x mult."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), K), dtype=np.uint16)
    for i, r in enumerate(rows):
        v = np.random.default_rng([seed, _TAG_ACT, int(r)]).standard_normal(K, dtype=np.float32)
        v *= np.float32(std)
        if outliers is not None and len(outliers):
            v[outliers] *= np.float32(mult)
        out[i] = bf16_bits(v)
    return out


def weight_rows(rows, K, seed, std):
    """BF16 bits of the given weight rows: N(0, std^2)."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), K), dtype=np.uint16)
    for i, r in enumerate(rows):
        v = np.random.default_rng([seed, _TAG_W, int(r)]).standard_normal(K, dtype=np.float32)
        out[i] = bf16_bits(v * np.float32(std))
    return out


def dense_inputs(name, rows_a=None, rows_w=None):
    """(A_bits, W_bits) for a dense workload, optionally only some rows."""
    c = WORKLOADS[name]
    K = c["K"]
    outl = outlier_channels(K, c["seed"], c["outlier_frac"], c["outlier_count"])
    ra = np.arange(c["M"]) if rows_a is None else rows_a
    rw = np.arange(c["N"]) if rows_w is None else rows_w
    A = act_rows(ra, K, c["seed"], c["act_std"], outl, c["outlier_mult"])
    W = weight_rows(rw, K, c["seed"], c["w_std"])
    return A, W


def rows_threaded(gen, rows, *args, threads=8):
    """gen(rows, *args) over row blocks on a thread pool (the per-row seeding
    makes the result independent of the split)."""
    from concurrent.futures import ThreadPoolExecutor
    rows = np.asarray(rows, dtype=np.int64)
    parts = np.array_split(rows, max(1, min(len(rows), threads * 4)))
    with ThreadPoolExecutor(threads) as ex:
        out = list(ex.map(lambda r: gen(r, *args), parts))
    return np.concatenate(out, axis=0)


def moe_routing(tokens, experts, topk, seed):
    """Top-k routing from N(0,1) logits (ties to the lower expert index).

    Returns (counts int64[E], offsets int32[E+1], token_of_row int64[sum]):
    rows are grouped by ascending expert, tokens ascending within an expert.
    """
    rng = np.random.default_rng([seed, _TAG_ROUTE])
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    # stable sort on -logit keeps the lower index first among equal logits
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    expert_of = order.reshape(-1)
    token_of = np.repeat(np.arange(tokens), topk)
    perm = np.lexsort((token_of, expert_of))
    counts = np.bincount(expert_of, minlength=experts).astype(np.int64)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets, token_of[perm]


def decode_counts(experts, lo, hi, seed):
    """Per-expert token counts uniform on {lo..hi}, and their offsets."""
    rng = np.random.default_rng([seed, _TAG_COUNTS])
    counts = rng.integers(lo, hi + 1, size=experts).astype(np.int64)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets


def expert_weight_torch(e, N, K, seed, std, device):
    """One expert's BF16 weight [N][K], drawn on the device with a seeded torch
    generator (used where a host generator would be too slow: 256 experts of
    4096 x 7168).  The returned bits are the shared input."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + int(e))
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    return (w * std).to(torch.bfloat16)
