"""Host logic of bench.py (CPU only): argument refusals, the streaming-ceiling
arithmetic behind roofline.stream_ceiling_GB_s, and the committed profile
records bench.py reads (well-formed, and measured on the current GEMM code)."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT,
                          env={**os.environ, "HIP_VISIBLE_DEVICES": ""})


@pytest.mark.parametrize("args", [("--gpus", "2"), ("--gpus", "8"),
                                  ("--mfma-scaled", "--workload", "moe"),
                                  ("--mfma-scaled", "--precise")])
def test_refused_arguments_exit_with_a_message(args):
    r = _run_bench(*args)
    assert r.returncode == 2, r.stderr
    assert "error" in json.loads(r.stdout.strip().splitlines()[-1])


def _rows(rate_of):
    """Synthetic ring-probe rows: the kernel's ring for every bucket at both
    loads, with weight rates from rate_of(act_rows, tiles_per_cu)."""
    rows = []
    for tiles in (16, 2):
        for ra, st in bench.GROUPED_BUCKETS:
            rows.append({"tiles_per_cu": tiles, "weights": "hbm", "act_rows": ra, "split": False,
                         "lds_reads": 0, "act_stages": st, "stages": st,
                         "weight_GB_s": rate_of(ra, tiles)})
    # rows the ceiling must ignore: other variants and regimes
    rows.append({"tiles_per_cu": 2, "weights": "hbm", "act_rows": 256, "split": True,
                 "lds_reads": 0, "act_stages": 2, "stages": 3, "weight_GB_s": 1.0})
    rows.append({"tiles_per_cu": 2, "weights": "hbm", "act_rows": 256, "split": False,
                 "lds_reads": 24, "act_stages": 2, "stages": 2, "weight_GB_s": 1.0})
    rows.append({"tiles_per_cu": 16, "weights": "l2", "act_rows": 128, "split": False,
                 "lds_reads": 0, "act_stages": 3, "stages": 3, "weight_GB_s": 1.0})
    return rows


def test_ring_ceilings_arithmetic():
    """With one rate R for every bucket the ceiling time is the workload's
    weight bytes over R; with per-bucket rates each expert's tiles take their
    bucket's rate (checked by a direct sum over the experts)."""
    R = 6000.0
    c = bench.ring_ceilings(_rows(lambda ra, t: R))
    for name in ("decode", "moe"):
        cfg = workloads.WORKLOADS[name]
        N, K = cfg["N"], cfg["K"]
        if name == "moe":
            counts = workloads.moe_routing(cfg["tokens"], cfg["experts"], cfg["topk"],
                                           cfg["seed"])[0]
        else:
            counts = workloads.decode_counts(cfg["experts"], cfg["m_lo"], cfg["m_hi"],
                                             cfg["seed"])[0]
        m_tiles = int(sum((int(m) + 255) // 256 for m in counts))
        t_us = m_tiles * N * K / (R * 1e3)
        assert c[name]["us"] == pytest.approx(t_us, rel=1e-12)
        assert sum(c[name]["m_tiles_per_bucket"].values()) == m_tiles
        ob = 4 if name == "moe" else 2
        gbytes = len(counts) * N * K * (1 + 4 / 16384) + counts.sum() * K * (1 + 4 / 128) \
            + counts.sum() * N * ob
        assert c[name]["GB_s"] == pytest.approx(gbytes / t_us / 1e3, rel=1e-12)

    def rate(ra, t):
        return 1000.0 * (1 + ra / 64) + (0 if t == 2 else 7.0)
    c = bench.ring_ceilings(_rows(rate))
    cfg = workloads.WORKLOADS["decode"]
    counts = workloads.decode_counts(cfg["experts"], cfg["m_lo"], cfg["m_hi"], cfg["seed"])[0]
    want = 0.0
    for m in counts:
        b = next(ra for ra, _ in bench.GROUPED_BUCKETS if int(m) <= ra)   # decode: m <= 256
        want += cfg["N"] * cfg["K"] / (rate(b, 2) * 1e3)
    assert c["decode"]["us"] == pytest.approx(want, rel=1e-12)


def test_profile_records_are_well_formed_and_current():
    """Every record line of profiles/*.md parses; the traffic and clock records
    carry the sha256 of the current GEMM code, so bench.py reports them (a
    change to the GEMM sources must come with new counter runs); the ceiling
    records are positive rates."""
    import glob
    digest = bench.kernel_source_digest()
    kinds = {}
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            for kind in ("traffic-record", "clock-record", "ceiling-record"):
                if line.startswith(kind + ":"):
                    rec = dict(kv.split("=", 1) for kv in line.split(":", 1)[1].split())
                    assert "kernel" in rec and "workload" in rec, line
                    kinds.setdefault(kind, []).append(rec)
                    if kind == "ceiling-record":
                        assert float(rec["GB_s"]) > 0
                    else:
                        assert rec["source_sha256"] == digest, \
                            f"{os.path.basename(path)}: {kind} of {rec['workload']} predates " \
                            f"the current GEMM code"
                    if kind == "traffic-record":
                        assert float(rec["bytes_per_launch"]) > 0
    for kind in ("traffic-record", "clock-record", "ceiling-record"):
        assert kinds.get(kind), f"no {kind} lines under profiles/"
    cfg = {"workload": "dense: whatever"}
    assert bench.recorded_traffic("fp8q_gemm", cfg) is not None
    assert bench.recorded_ceiling("fp8q_grouped_gemm", {"workload": "decode: x"}) is not None
    assert np.isfinite(bench.recorded_ceiling("fp8q_grouped_gemm", {"workload": "moe: x"}))
