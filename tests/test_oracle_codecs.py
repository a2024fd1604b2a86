"""Pins for the oracle's number formats (bf16 and OCP E4M3), CPU only.

The C oracle's encoders are checked against (a) exhaustive value tables and
nearest-value search in exact rational arithmetic (oracle/brute.py), and (b)
torch's own CPU casts, a library that shares nothing with either.
"""

import math
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import brute


def f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def f32_next(v: float, direction: int) -> float:
    return float(np.nextafter(np.float32(v), np.float32(math.copysign(math.inf, direction))))


# ------------------------------------------------------------------- E4M3 --

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), hex(c)
        else:
            assert got == ref[c], hex(c)


def test_e4m3_landmarks():
    # OCP E4M3: largest finite 448 = S.1111.110, smallest normal 2^-6 =
    # S.0001.000, smallest subnormal 2^-9 = S.0000.001, NaN = S.1111.111.
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0xFE) == -448.0
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(-448.0) == 0xFE
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80


def test_e4m3_roundtrip_all_finite_codes():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)


def _probe_values():
    vals, _ = brute._e4m3_table()
    fl = [float(v) for v in vals]
    out = set()
    for v in fl:
        out.add(v)
        out.add(f32_next(v, +1))
        out.add(f32_next(v, -1))
    for a, b in zip(fl, fl[1:]):
        mid = (a + b) / 2.0  # exact in float32: neighbours differ by one quantum
        assert f32(mid) == mid
        out.update([mid, f32_next(mid, +1), f32_next(mid, -1)])
    out.update([448.0, 449.0, 463.9, 464.0, 464.1, 480.0, 1e4, 3.4e38, math.inf,
                2.0 ** -10, 2.0 ** -11, 1e-30, 1e-45, 3 * 2.0 ** -11])
    return sorted(out)


def test_e4m3_encode_matches_table_search_at_every_midpoint():
    for v in _probe_values():
        for s in (v, -v):
            assert oracle.e4m3_encode(s) == brute.e4m3_encode(s), s


def test_e4m3_encode_random_against_table_search():
    rng = np.random.default_rng(123)
    mags = np.exp(rng.uniform(np.log(1e-5), np.log(600.0), 4000)).astype(np.float32)
    signs = np.where(rng.random(4000) < 0.5, -1.0, 1.0).astype(np.float32)
    for v in (mags * signs):
        assert oracle.e4m3_encode(float(v)) == brute.e4m3_encode(float(v)), float(v)


def test_e4m3_encode_matches_torch_cast_in_range():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even; values of
    # magnitude <= 448 never reach its (non-saturating) overflow path.
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.uniform(-448, 448, 50000),
        rng.standard_normal(50000) * 0.01,
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000),
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(a)) for a in v], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_saturates():
    for v in (448.5, 463.99, 464.0, 500.0, 1e9, math.inf):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE


# ------------------------------------------------------------------- bf16 --

def test_bf16_to_double_exhaustive():
    codes = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):   # signalling-NaN patterns widen to NaN
        ref = (codes << 16).view(np.float32).astype(np.float64)
    for c in range(0, 65536, 7):
        got = oracle.bf16_to_double(c)
        if math.isnan(ref[c]):
            assert math.isnan(got)
        else:
            assert got == ref[c]


def test_bf16_from_double_matches_torch_on_float32_values():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(30000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-39).astype(np.float32),   # bf16 subnormals
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
    ])
    # exact ties: float32 values whose low 16 bits are 0x8000
    ties = ((rng.integers(0x0080, 0x7F00, 5000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(a)) for a in v], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_bf16_from_double_matches_table_search_on_doubles():
    # doubles that are not float32 values (where a float32 detour would round
    # twice), including exact midpoints and one double-ulp either side of them
    rng = np.random.default_rng(5)
    vals, _ = brute._bf16_table()
    picks = rng.integers(1, len(vals) - 2, 600)
    probes = []
    for i in picks:
        a, b = vals[i], vals[i + 1]
        mid = (a + b) / 2
        probes += [float(mid), float(np.nextafter(float(mid), 0.0)), float(np.nextafter(float(mid), math.inf)),
                   float(a + (b - a) / 3), float(a + 2 * (b - a) / 3)]
    probes += list(rng.standard_normal(500) * 3.0)
    for p in probes:
        from fractions import Fraction
        for s in (p, -p):
            assert oracle.bf16_from_double(s) == brute.bf16_round(Fraction(s)), s


def test_bf16_from_double_signed_zero_and_nan():
    assert oracle.bf16_from_double(0.0) == 0x0000
    assert oracle.bf16_from_double(-0.0) == 0x8000
    assert (oracle.bf16_from_double(float("nan")) & 0x7F80) == 0x7F80
    assert oracle.bf16_from_double(1e300) == 0x7F80
