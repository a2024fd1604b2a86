"""Pure-Python brute force for tiny inputs -- TEST INFRASTRUCTURE ONLY.

These functions pin the C oracle (``ep_oracle.c``) by a different route:

* number formats are handled by *enumeration*: every finite non-negative
  bf16 / E4M3 value is listed exactly (``fractions.Fraction``) and rounding
  picks the nearest listed value, ties to the even code;
* layout counts earlier equal keys pair by pair, straight from the
  definition of a stable expert-grouped (expanded) layout;
* combine sums exact rationals and rounds once.

They are far too slow for anything but tiny shapes.
"""

from __future__ import annotations

import bisect
from fractions import Fraction
from functools import lru_cache
from typing import List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------- format tables --


@lru_cache(maxsize=None)
def _e4m3_table() -> Tuple[List[Fraction], List[int]]:
    """All finite non-negative OCP E4M3 values with their codes, ascending.

    Field layout S.EEEE.MMM, bias 7; exponent field 0 is subnormal with an
    implicit leading 0 and exponent 1 - bias; S.1111.111 is NaN; there is no
    infinity, so S.1111.110 = 1.75 * 2^8 = 448 is the largest finite value.
    """
    vals, codes = [], []
    for code in range(0x00, 0x80):
        ef, mf = code >> 3, code & 7
        if ef == 15 and mf == 7:
            continue
        if ef == 0:
            v = Fraction(mf, 8) * Fraction(2) ** (1 - 7)
        else:
            v = (1 + Fraction(mf, 8)) * Fraction(2) ** (ef - 7)
        vals.append(v)
        codes.append(code)
    return vals, codes


@lru_cache(maxsize=None)
def _e5m2_table() -> Tuple[List[Fraction], List[int]]:
    """All finite non-negative OCP E5M2 values with their codes, ascending.

    Field layout S.EEEEE.MM, bias 15; exponent field 0 is subnormal
    (exponent 1 - bias, implicit 0); exponent field 31 holds infinity and
    NaNs, so S.11110.11 = 1.75 * 2^15 = 57344 is the largest finite value.
    """
    vals, codes = [], []
    for code in range(0x00, 0x7C):
        ef, mf = code >> 2, code & 3
        v = Fraction(mf, 4) * Fraction(2) ** (1 - 15) if ef == 0 else \
            (1 + Fraction(mf, 4)) * Fraction(2) ** (ef - 15)
        vals.append(v)
        codes.append(code)
    return vals, codes


def e5m2_encode(v: float) -> int:
    """Nearest E5M2 code to v (saturating to +-57344), by table."""
    if v != v:
        return 0x7F
    neg = np.signbit(np.float64(v))
    vals, codes = _e5m2_table()
    if np.isinf(v):
        return codes[-1] | (0x80 if neg else 0)
    c = _nearest_code(abs(Fraction(float(v))), vals, codes)
    return c | (0x80 if neg else 0)


@lru_cache(maxsize=None)
def _bf16_table() -> Tuple[List[Fraction], List[int]]:
    """All finite non-negative bf16 values with their codes, ascending
    (8 exponent bits with bias 127, 7 stored mantissa bits)."""
    vals, codes = [], []
    for code in range(0x0000, 0x7F80):
        ef, mf = code >> 7, code & 0x7F
        if ef == 0:
            v = Fraction(mf, 128) * Fraction(2) ** (1 - 127)
        else:
            v = (1 + Fraction(mf, 128)) * Fraction(2) ** (ef - 127)
        vals.append(v)
        codes.append(code)
    return vals, codes


def _nearest_code(a: Fraction, vals: Sequence[Fraction], codes: Sequence[int]) -> int:
    """Code of the listed value nearest to a >= 0, ties to the even code;
    a beyond the largest value gives the largest value (saturation)."""
    i = bisect.bisect_left(vals, a)
    if i == 0:
        return codes[0]
    if i == len(vals):
        return codes[-1]
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = a - lo, hi - a
    if dlo < dhi:
        return codes[i - 1]
    if dhi < dlo:
        return codes[i]
    return codes[i - 1] if codes[i - 1] % 2 == 0 else codes[i]


def e4m3_value(code: int) -> Optional[Fraction]:
    """Exact value of an E4M3 code, None for NaN."""
    vals, codes = _e4m3_table()
    mag = code & 0x7F
    if mag == 0x7F:
        return None
    v = vals[codes.index(mag)]
    return -v if code & 0x80 else v


def e4m3_encode(v: float) -> int:
    """Nearest E4M3 code to the float v (saturating to +-448), by table."""
    if v != v:
        return 0x7F
    neg = np.signbit(np.float64(v))
    vals, codes = _e4m3_table()
    if np.isinf(v):
        return codes[-1] | (0x80 if neg else 0)
    c = _nearest_code(abs(Fraction(float(v))), vals, codes)
    return c | (0x80 if neg else 0)


def bf16_value(code: int) -> Fraction:
    vals, codes = _bf16_table()
    mag = code & 0x7FFF
    v = vals[mag]
    return -v if code & 0x8000 else v


def bf16_round(q: Fraction, negative_zero: bool = False) -> int:
    """Nearest bf16 code to the exact rational q (no overflow expected)."""
    vals, codes = _bf16_table()
    if q == 0:
        return 0x8000 if negative_zero else 0
    c = _nearest_code(abs(q), vals, codes)
    if c == codes[-1] and abs(q) > vals[-1]:
        raise OverflowError("value beyond the bf16 range")
    return c | (0x8000 if q < 0 else 0)


# ------------------------------------------------------------------ layout --

def layout(topk_idx: np.ndarray, E: int, alignment: int = 1, capacity: int = 0):
    """Expanded, expert-grouped, stable layout straight from its definition:
    slot(i) = start(e) + #{i' < i : key(i') == e}.  Packed: start(e) is the
    sum over experts below e of their counts rounded up to `alignment`.
    Fixed stride: start(e) = e * capacity and a pair whose rank reaches the
    capacity is dropped.  Returns (counts, offsets, slot, src, invalid,
    dropped)."""
    idx = [int(v) for v in np.asarray(topk_idx).reshape(-1)]
    T, k = np.asarray(topk_idx).shape
    valid = [0 <= e < E for e in idx]
    raw = [sum(1 for e, ok in zip(idx, valid) if ok and e == x) for x in range(E)]
    if capacity > 0:
        starts = [x * capacity for x in range(E)]
        counts = [min(c, capacity) for c in raw]
        total = E * capacity
    else:
        starts, total = [], 0
        for x in range(E):
            starts.append(total)
            total += -(-raw[x] // alignment) * alignment
        counts = raw
    slot, dropped = [], 0
    for i, (e, ok) in enumerate(zip(idx, valid)):
        if not ok:
            slot.append(-1)
            continue
        earlier = sum(1 for i2 in range(i) if valid[i2] and idx[i2] == e)
        if capacity > 0 and earlier >= capacity:
            slot.append(-1)
            dropped += 1
            continue
        slot.append(starts[e] + earlier)
    src = [-1] * max(total, T * k)
    for i, r in enumerate(slot):
        if r >= 0:
            src[r] = i // k
    invalid = sum(1 for e in idx if not (e == -1 or 0 <= e < E))
    return (np.array(counts, np.int32), np.array(starts + [total], np.int32),
            np.array(slot, np.int32).reshape(T, k), np.array(src, np.int32), invalid, dropped)


# ---------------------------------------------------------------- dispatch --

def fp8_quantize_row(x_bits: np.ndarray):
    """Per 128-channel block: amax (exact, NaN ignored), scale =
    float32(amax / 448), code = nearest E4M3 of float32(x / scale); a NaN
    quotient gives S.1111.111 with the sign of x.  Returns (codes, scales)."""
    H = x_bits.shape[0]
    xs = [_bf16_float(int(b)) for b in x_bits]
    codes, scales = [], []
    for b in range(H // 128):
        blk = xs[b * 128:(b + 1) * 128]
        amax = np.float32(max((abs(v) for v in blk if v == v), default=0.0))
        scale = np.float32(amax / np.float32(448.0))
        scales.append(float(scale))
        for v in blk:
            if amax == 0:
                codes.append(0)
                continue
            with np.errstate(invalid="ignore"):
                q = np.float32(np.float32(v) / scale)
            if q != q:   # NaN quotient: S.1111.111 with the sign of x
                codes.append(0x7F | (0x80 if np.signbit(np.float32(v)) else 0))
            else:
                codes.append(e4m3_encode(float(q)))
    return np.array(codes, np.uint8), np.array(scales, np.float32)


def _bf16_float(code: int) -> float:
    """bf16 code -> Python float, including infinities and NaN."""
    if (code & 0x7F80) == 0x7F80:
        if code & 0x7F:
            return float("nan") if not code & 0x8000 else -float("nan")
        return -float("inf") if code & 0x8000 else float("inf")
    return float(bf16_value(code))


def quantize_row(x_bits: np.ndarray, fmt: str = "e4m3", scale: str = "fp32"):
    """Per 128-channel block, for every format and scale mode, from the
    definitions with exact rationals where they decide: the power-of-two
    exponent is the smallest integer e with 2^e >= amax / max_finite
    (compared exactly), UE8M0 clamps e to -127; q = x * 2^-e is exact.
    Returns (codes, scales as float32 or uint8)."""
    H = x_bits.shape[0]
    xs = [_bf16_float(int(b)) for b in x_bits]
    fmax = 448 if fmt == "e4m3" else 57344
    enc = e4m3_encode if fmt == "e4m3" else e5m2_encode
    codes, scales = [], []
    for b in range(H // 128):
        blk = xs[b * 128:(b + 1) * 128]
        amax = max((abs(v) for v in blk if v == v), default=0.0)
        if amax == 0:
            codes += [0] * 128
            scales.append(0.0 if scale != "ue8m0" else 0)
            continue
        if scale == "fp32" or amax == float("inf"):
            s = np.float32(np.float32(amax) / np.float32(fmax))
            scales.append(float(s) if scale != "ue8m0" else 0xFF)
            for v in blk:
                with np.errstate(invalid="ignore"):
                    q = np.float32(np.float32(v) / s)
                codes.append(0x7F | (0x80 if np.signbit(np.float32(v)) else 0) if q != q else enc(float(q)))
            continue
        ratio = Fraction(amax) / fmax
        e = 0
        while Fraction(2) ** e < ratio:
            e += 1
        while Fraction(2) ** (e - 1) >= ratio:
            e -= 1
        if scale == "ue8m0":
            e = max(e, -127)
            scales.append(e + 127)
        else:
            scales.append(float(Fraction(2) ** e))
        for v in blk:
            if v != v:
                codes.append(0x7F | (0x80 if np.signbit(np.float32(v)) else 0))
            else:
                codes.append(enc(float(Fraction(v) / Fraction(2) ** e)))
    return np.array(codes, np.uint8), np.array(scales, np.uint8 if scale == "ue8m0" else np.float32)


# ----------------------------------------------------------------- combine --

def combine(y_bits: np.ndarray, slot: np.ndarray, w: Optional[np.ndarray]) -> np.ndarray:
    """out[t,c] = round_bf16( exact sum_j w[t,j] * y[slot[t,j], c] )."""
    T, k = slot.shape
    H = y_bits.shape[1]
    out = np.zeros((T, H), np.uint16)
    for t in range(T):
        for c in range(H):
            acc = Fraction(0)
            for j in range(k):
                r = int(slot[t, j])
                if r < 0:
                    continue
                wt = Fraction(1) if w is None else Fraction(float(w[t, j]))
                acc += wt * bf16_value(int(y_bits[r, c]))
            out[t, c] = bf16_round(acc)
    return out
