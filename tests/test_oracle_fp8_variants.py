"""Pins for the oracle's 8-bit float variants, CPU only: the OCP E5M2
codec, power-of-two (round_scale) and UE8M0 scales for both formats, and
the dispatch of pre-quantized input.

Routes: torch's float8_e5m2 dtype (library special case); exhaustive value
tables with exact rational nearest search (oracle/brute.py); a quantiser
whose power-of-two exponent comes from exact rational comparisons instead
of the fp32 quotient; hand-worked blocks (tests/golden/fp8_variants_handworked.txt).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from combine_ep_layout_04_amd.inputs import (
    WORKLOADS, bf16_bits_from_float32, float32_from_bf16_bits, make_inputs, make_random_case,
)

from golden_io import read_cases


def test_e5m2_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e5m2_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), hex(c)
        else:
            assert got == ref[c], hex(c)


def test_e5m2_encode_vs_table_and_torch():
    vals, _ = brute._e5m2_table()
    probes = set()
    fl = [float(v) for v in vals]
    for a, b in zip(fl, fl[1:]):
        mid = (a + b) / 2
        probes.update([a, mid, float(np.nextafter(np.float32(mid), np.float32(0))),
                       float(np.nextafter(np.float32(mid), np.float32(1e9)))])
    probes.update([57344.0, 60000.0, 61440.0, 1e9, math.inf, 2.0 ** -17, 2.0 ** -18, 3 * 2.0 ** -18])
    for v in probes:
        for sv in (v, -v):
            assert oracle.e5m2_encode(sv) == brute.e5m2_encode(sv), sv
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-57344, 57344, 30000), rng.standard_normal(30000) * 1e-3]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = np.array([oracle.e5m2_encode(float(a)) for a in v], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("case", read_cases("fp8_variants_handworked.txt"), ids=lambda c: c["name"])
def test_fp8_variants_handworked(case):
    fmt = case["format"][0]
    xf = np.zeros(128, np.float32)
    xf[:len(case["x"])] = case["x"]
    xb = bf16_bits_from_float32(xf)
    assert np.array_equal(float32_from_bf16_bits(xb), xf)
    slot = np.array([[0]], np.int32)
    want = np.zeros(128, np.uint8)
    want[:len(case["codes"])] = case["codes"]
    for mode, key in (("fp32", "scale_fp32"), ("pow2", "scale_pow2"), ("ue8m0", "scale_ue8m0")):
        if key not in case:
            continue
        q, sc, _ = oracle.dispatch_quant(xb[None, :], slot, fmt=fmt, scale=mode)
        np.testing.assert_array_equal(q[0], want)
        assert sc[0, 0] == case[key][0]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("mode", ["fp32", "pow2", "ue8m0"])
def test_dispatch_quant_vs_bruteforce(fmt, mode):
    inp = make_random_case(41, 6, 384, 4, 2, mask_frac=0.2)
    x = float32_from_bf16_bits(inp.x_bits).copy()
    x[0, :128] = 0.0                              # zero block
    x[1, 128:256] *= 1e-30                        # tiny amax (UE8M0 clamps)
    x[2, 5] = np.inf                              # infinite amax
    x[3, 200] = np.nan                            # NaN ignored by amax
    x[4, :128] *= 1e20                            # huge amax
    x[5, 256:] = 0.5                              # amax a power of two
    xb = bf16_bits_from_float32(x)
    L = oracle.layout(inp.topk_idx, 4)
    q, sc, _ = oracle.dispatch_quant(xb, L.slot, fmt=fmt, scale=mode)
    for t in range(6):
        bq, bs = brute.quantize_row(xb[t], fmt, mode)
        for j in range(2):
            r = L.slot[t, j]
            if r >= 0:
                np.testing.assert_array_equal(q[r], bq)
                np.testing.assert_array_equal(sc[r].view(np.uint8), bs.view(np.uint8))


def _exact_pow2_exponent(amax: float, fmax: float) -> int:
    """Smallest e with 2^e >= amax / fmax, by exact rational comparisons."""
    from fractions import Fraction
    r = Fraction(amax) / Fraction(fmax)
    e = r.numerator.bit_length() - r.denominator.bit_length()
    while Fraction(2) ** e < r:
        e += 1
    while Fraction(2) ** (e - 1) >= r:
        e -= 1
    return e


@pytest.mark.parametrize("fmt,fmax", [("e4m3", 448.0), ("e5m2", 57344.0)])
def test_pow2_exponent_every_bf16_amax(fmt, fmax):
    # every finite positive bf16 magnitude as the amax of one block (the
    # block is [amax, -amax, 0, ...]): the power-of-two scale is the exact
    # smallest 2^e >= amax / fmax, so amax * 2^-e lies in (fmax / 2, fmax]
    # and its code (rounding is monotone, fmax / 2 and fmax are codes)
    # decodes to a value in [fmax / 2, fmax]: it never saturates; with UE8M0
    # the exponent is the same clamped at -127
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    xb = np.zeros((bits.size, 128), np.uint16)
    xb[:, 0] = bits
    xb[:, 1] = bits | 0x8000
    slot = np.arange(bits.size, dtype=np.int32)[:, None]
    q, sc, _ = oracle.dispatch_quant(xb, slot, fmt=fmt, scale="pow2")
    qb, sb, _ = oracle.dispatch_quant(xb, slot, fmt=fmt, scale="ue8m0")
    amax = float32_from_bf16_bits(bits).astype(np.float64)
    want = np.array([_exact_pow2_exponent(a, fmax) for a in amax])
    got = np.frexp(sc[:, 0].astype(np.float64))[1] - 1
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(sb[:, 0].astype(np.int64), np.maximum(want, -127) + 127)
    dec = oracle.e5m2_decode if fmt == "e5m2" else oracle.e4m3_decode
    v = np.array([dec(int(c)) for c in q[:, 0]])
    assert np.all((v >= fmax / 2) & (v <= fmax))
    np.testing.assert_array_equal(q[:, 1], q[:, 0] | 0x80)


def test_dispatch_quant_e4m3_fp32_is_dispatch_fp8():
    inp = make_inputs(WORKLOADS["fp8"], T=96)
    L = oracle.layout(inp.topk_idx, 256)
    q1, s1, _ = oracle.dispatch_fp8(inp.x_bits, L.slot)
    q2, s2, _ = oracle.dispatch_quant(inp.x_bits, L.slot, fmt="e4m3", scale="fp32")
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("fmt,fmax", [("e4m3", 448.0), ("e5m2", 57344.0)])
def test_pow2_scale_vs_torch_cast(fmt, fmax):
    # library special case: with the scale a power of two the quotient is
    # exact, so torch's RNE cast of x * 2^-e is the code (in range)
    inp = make_inputs(WORKLOADS["fp8"], T=64)
    slot = np.arange(64, dtype=np.int32)[:, None]
    q, sc, _ = oracle.dispatch_quant(inp.x_bits, slot, fmt=fmt, scale="pow2")
    xf = float32_from_bf16_bits(inp.x_bits).reshape(64, -1, 128).astype(np.float64)
    qf = (xf / sc[:, :, None].astype(np.float64)).reshape(64, -1).astype(np.float32)
    assert np.abs(qf).max() <= fmax
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    ref = torch.from_numpy(qf).to(dt).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, ref)
    # and the scale is the smallest power of two at or above amax / fmax
    amax = np.abs(xf).max(axis=2)
    assert np.all(sc >= amax / fmax) and np.all(sc / 2 < amax / fmax)


def test_dispatch_prequant_is_a_copy():
    inp = make_random_case(51, 40, 256, 8, 3, mask_frac=0.2, dup_frac=1.0)
    L = oracle.layout(inp.topk_idx, 8)
    rng = np.random.default_rng(52)
    xq = rng.integers(0, 256, (40, 256), dtype=np.uint8)
    xs = rng.standard_normal((40, 2)).astype(np.float32)
    q, sc, rw = oracle.dispatch_prequant(xq, xs, L.slot, inp.topk_weights)
    t, j = np.nonzero(L.slot >= 0)
    np.testing.assert_array_equal(q[L.slot[t, j]], xq[t])
    np.testing.assert_array_equal(sc[L.slot[t, j]], xs[t])
    np.testing.assert_array_equal(rw[L.slot[t, j]], inp.topk_weights[t, j])
    assert not q[L.n:].any()
