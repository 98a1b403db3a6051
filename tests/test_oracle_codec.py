"""Pins for the oracle's E4M3 codec (CPU only).

Pinned against: hand-derived landmark values (tests/golden/e4m3_landmarks.txt,
worked out from the format definition), a brute-force nearest search, and the
float8_e4m3fn conversion of PyTorch (an independent library routine).
"""

import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_landmarks.txt")


def _golden():
    dec, enc = [], []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        kind, a, b = line.split()
        if kind == "decode":
            dec.append((int(a, 16), float(b)))
        else:
            enc.append((float(a), int(b, 16)))
    return dec, enc


def test_decode_landmarks():
    dec, _ = _golden()
    assert len(dec) >= 10
    for code, val in dec:
        got = e4m3.DECODE_TABLE[code]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_encode_landmarks():
    _, enc = _golden()
    assert len(enc) >= 8
    vals = np.array([v for v, _ in enc])
    codes = e4m3.encode(vals)
    for (v, c), got in zip(enc, codes):
        assert got == c, (v, hex(c), hex(got))


def test_decode_table_structure():
    t = e4m3.DECODE_TABLE
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    assert np.array_equal(-t[0x80:0xFF], pos) or np.array_equal(np.abs(t[0x80:0xFF]), pos)
    assert np.all(np.signbit(t[0x80:0xFF]))
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    assert e4m3.MAX_FINITE == 448.0
    # every value is a multiple of 2^-9 with at most 4 significant bits
    iv = pos * 512
    assert np.all(iv == np.round(iv))
    for v in iv[1:]:
        v = int(v)
        while v % 2 == 0:
            v //= 2
        assert v < 16


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_encode_all_bf16_vs_bruteforce():
    v = _all_bf16_finite()
    assert np.array_equal(e4m3.encode(v), e4m3.nearest_bruteforce(v))


def _midpoint_sweep():
    pos = e4m3.DECODE_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)  # exact in fp32
    pts = [mids, pos.astype(np.float32)]
    for d in (1, 2, 3):
        pts.append(np.nextafter(mids, np.float32(np.inf)))
        pts.append(np.nextafter(mids, np.float32(0)))
        mids = pts[-2]
    v = np.concatenate(pts)
    return np.concatenate([v, -v])


def test_encode_midpoints_and_random_fp32_vs_bruteforce():
    rng = np.random.default_rng(7)
    # random fp32 bit patterns restricted to |v| <= 512, plus the midpoint sweep
    bits = rng.integers(0, 2**31, size=400_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 512)]
    u = rng.uniform(-460, 460, size=200_000).astype(np.float32)
    v = np.concatenate([v, u, _midpoint_sweep()])
    assert np.array_equal(e4m3.encode(v), e4m3.nearest_bruteforce(v))


def test_encode_matches_torch_float8_in_range():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        _all_bf16_finite(),
        _midpoint_sweep(),
        rng.uniform(-448, 448, size=300_000).astype(np.float32),
        (rng.standard_normal(300_000) * 2.0 ** rng.integers(-20, 8, 300_000)).astype(np.float32),
    ])
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(v), ref)


def test_encode_decode_roundtrip_and_signed_zero():
    codes = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], dtype=np.uint8)
    back = e4m3.encode(e4m3.decode(codes))
    assert np.array_equal(back, codes)
    assert e4m3.encode(np.array([-0.0]))[0] == 0x80
    assert e4m3.encode(np.array([-1e-30]))[0] == 0x80
    assert e4m3.encode(np.array([0.0]))[0] == 0x00


def test_encode_rejects_nonfinite():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.inf]))
