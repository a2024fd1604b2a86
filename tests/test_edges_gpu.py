"""GPU edge cases against the oracle: empty, masked, invalid and duplicate
routing, ragged and extreme shapes, a single hot expert, determinism and a
non-default stream.

Combine here reduces random mixed-sign expert outputs, so besides the final
bf16 rounding the fp32 accumulation error enters; the tolerance is one bf16
ulp of the oracle value plus the bound for k fused multiply-adds in fp32,
2 * k * 2^-24 * sum_j |w_j y_j| (written in ``combine_tolerance``).
"""

import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_04_amd import ep
from combine_ep_layout_04_amd.inputs import (
    bf16_bits_from_float32, float32_from_bf16_bits, make_gradient, make_random_case,
)

from gpu_util import DEV, bf16_bits, bf16_ulp, dev, host, x_dev

pytestmark = pytest.mark.gpu


def combine_tolerance(y_bits, slot, w, ref_bits):
    T, k = slot.shape
    yf = float32_from_bf16_bits(y_bits).astype(np.float64)
    s = np.zeros((T, y_bits.shape[1]))
    for j in range(k):
        r = slot[:, j]
        ok = r >= 0
        wj = np.ones(T) if w is None else w[:, j].astype(np.float64)
        s[ok] += np.abs(wj[ok, None] * yf[r[ok]])
    ref = float32_from_bf16_bits(ref_bits).astype(np.float64)
    return bf16_ulp(ref) + 2.0 * k * 2.0 ** -24 * s


def run_case(idx, x_bits, w, E, y_bits=None, fp8=None, stream=None, use_weights=True):
    """Everything through the C ABI, outputs pre-filled with sentinels;
    returns host copies.  The oracle's layout is computed first and its N
    sizes nothing on the GPU side (capacity is always T*k rows)."""
    T, k = idx.shape
    H = x_bits.shape[1]
    P = T * k
    fp8 = (H % 128 == 0) if fp8 is None else fp8
    if stream is not None:
        # inputs and sentinel fills are made on torch's current stream
        torch.cuda.synchronize()
    idx_d = dev(idx)
    x_d = x_dev(x_bits)
    w_d = dev(w) if (w is not None and use_weights) else None
    src = torch.full((P,), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((T, k), -9, dtype=torch.int32, device=DEV)
    recv = torch.full((P, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    rw = torch.full((P,), float("nan"), dtype=torch.float32, device=DEV) if w_d is not None else None
    if fp8:
        q = torch.full((P, H), 0xEE, dtype=torch.uint8, device=DEV)
        s = torch.full((P, H // 128), float("nan"), dtype=torch.float32, device=DEV)
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())
    counts, offsets, slot, src, inval = ep.ep_layout(idx_d, E, slot=slot, src=src, stream=stream)
    ep.ep_dispatch(x_d, slot, w_d, recv_x=recv, recv_weights=rw, stream=stream)
    g = {}
    if fp8:
        ep.ep_dispatch(x_d, slot, None, fp8=True, recv_x=q, recv_scales=s, stream=stream)
    out = None
    if y_bits is not None:
        out = torch.full((T, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        y_d = x_dev(y_bits)
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        ep.ep_combine(y_d, slot, w_d, out=out, stream=stream)
    if stream is not None:
        stream.synchronize()
    torch.cuda.synchronize()
    g.update(counts=host(counts), offsets=host(offsets), slot=host(slot), src=host(src),
             inval=int(host(inval)[0]), recv=bf16_bits(recv),
             rw=None if rw is None else host(rw))
    if fp8:
        g.update(q=host(q), s=host(s))
    if out is not None:
        g["out"] = bf16_bits(out)
    return g


def check_case(idx, x_bits, w, E, seed=0, use_weights=True, stream=None):
    T, k = idx.shape
    H = x_bits.shape[1]
    rng = np.random.default_rng(seed)
    y = bf16_bits_from_float32(rng.standard_normal((T * k, H)).astype(np.float32))
    print(f"[edges] T={T} k={k} E={E} H={H}", flush=True)
    g = run_case(idx, x_bits, w, E, y_bits=y, stream=stream, use_weights=use_weights)
    L = oracle.layout(idx, E)
    n = L.n
    np.testing.assert_array_equal(g["counts"], L.counts)
    np.testing.assert_array_equal(g["offsets"], L.offsets)
    np.testing.assert_array_equal(g["slot"], L.slot)
    np.testing.assert_array_equal(g["src"][:n], L.src[:n])
    assert np.all(g["src"][n:] == -7)
    assert g["inval"] == L.num_invalid
    wo = w if use_weights else None
    recv, rw = oracle.dispatch_bf16(x_bits, L.slot, wo)
    np.testing.assert_array_equal(g["recv"][:n], recv[:n])
    assert np.all(g["recv"][n:] == 0xFFFF)
    if rw is not None:
        np.testing.assert_array_equal(g["rw"][:n], rw[:n])
        assert np.all(np.isnan(g["rw"][n:]))
    if "q" in g:
        q, s, _ = oracle.dispatch_fp8(x_bits, L.slot)
        np.testing.assert_array_equal(g["q"][:n], q[:n])
        np.testing.assert_array_equal(g["s"][:n].view(np.uint32), s[:n].view(np.uint32))
        assert np.all(g["q"][n:] == 0xEE)
    ref = oracle.combine(y, L.slot, wo)
    got = (g["out"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = (ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    tol = combine_tolerance(y, L.slot, wo, ref)
    bad = np.abs(got - want) > tol
    assert not bad.any(), f"combine off at {np.argwhere(bad)[:5].tolist()}"
    return g, L


@pytest.mark.parametrize("T,k,E,H", [
    (1, 1, 1, 8),          # smallest everything
    (3, 2, 4, 16),
    (1000, 3, 7, 200),     # ragged chunk (3000 pairs), 25-vector rows, tail-only dispatch
    (513, 5, 33, 1032),    # 129-vector rows: one pass + a one-vector tail
    (300, 9, 40, 256),     # k = 9: the generic combine loop
    (64, 64, 64, 128),     # k = EP_MAX_TOPK
    (2048, 4, 1024, 256),  # E = EP_MAX_EXPERTS
    (16, 2, 8, 65536),     # hidden = EP_MAX_HIDDEN
    (40000, 8, 1024, 8),   # 320000 pairs: 1280-pair chunks, 250 of them
    (65537, 8, 256, 8),    # 524296 pairs: 2304-pair chunks, a ragged last one
    # rows shorter than k lanes: the slots of lanes past the row end are
    # still read (by readlane) while only the row's lanes have work
    (129, 8, 16, 24),      # 3-vector rows, 8 slots
    (77, 12, 16, 24),      # 3-vector rows, k = 12: the generic combine loop
    (40, 40, 64, 520),     # 65-vector rows: a one-vector tail past 64 lanes, k = 40
    # whole-tile rows under 512 vectors in dispatches that write >= 2^23
    # vectors: the tiled dispatch
    (8192, 4, 64, 2048),   # 256-vector rows, one slot group
    (6144, 8, 256, 3072),  # 384-vector rows, two slot groups
    # 64-lane tiles, where the last 128-lane tile would be at most half full
    (300, 9, 40, 1536),    # combine, 192 vectors: three full tiles, k = 9 (generic loop)
    (257, 8, 64, 1152),    # combine, 144 vectors: tiles of 64, 64 and 16
    (257, 6, 40, 3584),    # dispatch and combine, 448 vectors: seven full tiles
    (129, 8, 16, 3200),    # dispatch and combine, 400 vectors: the last tile of 16 lanes
    (333, 12, 32, 2176),   # cast, 136 units: tiles of 64, 64 and 8, three slot groups
    (200, 3, 16, 2944),    # cast, 184 units: tiles of 64, 64 and 56
    (130, 8, 32, 5120),    # cast, 320 units: five full tiles, two slot groups
])
def test_shapes(T, k, E, H):
    inp = make_random_case(T * 31 + k, T, H, E, k, mask_frac=0.1, dup_frac=0.0 if k <= E else 1.0)
    check_case(inp.topk_idx, inp.x_bits, inp.topk_weights, E, seed=T)


def test_masked_invalid_and_duplicates():
    inp = make_random_case(7, 777, 384, 16, 6, mask_frac=0.3, dup_frac=1.0, invalid_frac=0.1)
    g, L = check_case(inp.topk_idx, inp.x_bits, inp.topk_weights, 16)
    assert L.num_invalid > 0 and g["inval"] == L.num_invalid


def test_all_masked():
    inp = make_random_case(8, 50, 256, 8, 4)
    idx = np.full_like(inp.topk_idx, -1)
    g, L = check_case(idx, inp.x_bits, inp.topk_weights, 8)
    assert L.n == 0 and not g["counts"].any() and not g["offsets"].any()
    assert not g["out"].any()          # every token reduces the empty sum to +0
    assert np.all(g["recv"] == 0xFFFF)  # nothing dispatched


def test_single_hot_expert():
    # every pair to one expert: one LDS counter and one bit-matrix row take
    # every update, and the stable order must still be the flat order
    T, k, E, H = 4096, 8, 256, 128
    inp = make_random_case(9, T, H, E, k)
    idx = np.full((T, k), 37, dtype=np.int64)
    idx[::5, 3] = -1
    check_case(idx, inp.x_bits, inp.topk_weights, E)


def test_unit_weights():
    inp = make_random_case(10, 700, 512, 12, 3, mask_frac=0.2)
    check_case(inp.topk_idx, inp.x_bits, inp.topk_weights, 12, use_weights=False)


def test_fp8_special_blocks():
    # zero blocks, negative zeros, subnormal-range values, huge outliers,
    # both sides of the fast-quotient threshold, infinities and NaNs
    inp = make_random_case(11, 40, 512, 8, 2)
    x = float32_from_bf16_bits(inp.x_bits).copy()
    x[0, :128] = 0.0
    x[1, 128:256] = -0.0
    x[2, :] *= 1e-30
    x[3, 5] = 3e38
    x[4, 300] = -1e-38
    x[5, :128] = 1.0
    x[5, 7] = 3.5
    x[6, :128] = 0.0
    x[6, 3] = 1e-38        # a block whose amax is an fp32 denormal
    x[6, 9] = -2e-39
    # either side of the fast-quotient threshold amax = 2^-80
    x[7, :128] = np.float32(2.0 ** -83) * x[7, :128] / np.abs(x[7, :128]).max()
    x[7, 5] = 2.0 ** -80
    x[7, 128:256] = np.float32(2.0 ** -84) * x[7, 128:256] / np.abs(x[7, 128:256]).max()
    x[7, 130] = -(2.0 ** -80) * (1 - 2.0 ** -8)
    # non-finite blocks: infinities (amax = inf) and NaNs (ignored by amax)
    x[8, 3] = np.inf
    x[8, 4] = -np.inf
    x[8, 260] = np.nan
    x[9, :128] = np.nan
    x[9, 200] = -np.inf
    xb = bf16_bits_from_float32(x)
    xb[8, 261] = 0xFFC0    # a negative NaN
    check_case(inp.topk_idx, xb, inp.topk_weights, 8)


def test_zero_tokens():
    counts, offsets, slot, src, inval = ep.ep_layout(torch.empty((0, 4), dtype=torch.int64, device=DEV), 16)
    torch.cuda.synchronize()
    assert not host(counts).any() and not host(offsets).any() and int(host(inval)[0]) == 0
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    recv, _, _ = ep.ep_dispatch(x, slot)
    out = ep.ep_combine(recv, slot, None)
    assert recv.shape == (0, 256) and out.shape == (0, 256)


def test_zero_tokens_every_entry_point():
    # T = 0 through the layout variants, the 8-bit casts, the pre-quantized
    # copy and both backward passes: no rows, and the layouts' count and
    # offset arrays as the oracle gives them for an empty batch
    idx0 = np.empty((0, 4), dtype=np.int64)
    for A, cap in ((1, 0), (16, 0), (1, 8)):
        nd = torch.full((1,), -5, dtype=torch.int32, device=DEV)
        counts, offsets, slot, src, inval = ep.ep_layout(dev(idx0), 16, alignment=A, capacity=cap,
                                                         num_dropped=nd if cap else None)
        torch.cuda.synchronize()
        L = oracle.layout(idx0, 16, alignment=A, capacity=cap)
        np.testing.assert_array_equal(host(counts), L.counts)
        np.testing.assert_array_equal(host(offsets), L.offsets)
        assert int(host(inval)[0]) == 0
        if cap:
            assert int(host(nd)[0]) == 0
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    slot = torch.empty((0, 4), dtype=torch.int32, device=DEV)
    for fmt, mode in (("e4m3", "fp32"), ("e5m2", "ue8m0")):
        q, s, _ = ep.ep_dispatch(x, slot, None, fp8=True, fmt=fmt, scale=mode)
        assert q.shape == (0, 256) and s.shape[0] == 0
    q, s, _ = ep.ep_dispatch_prequantized(torch.empty((0, 256), dtype=torch.uint8, device=DEV),
                                          torch.empty((0, 2), dtype=torch.float32, device=DEV), slot)
    gy, gw = ep.ep_combine_backward(x, torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), slot, None)
    gx, gxw = ep.ep_dispatch_backward(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV),
                                      torch.empty(0, dtype=torch.float32, device=DEV), slot)
    torch.cuda.synchronize()
    assert q.shape == (0, 256) and gy.shape == (0, 256) and gw.shape == (0, 4)
    assert gx.shape == (0, 256) and gxw.shape == (0, 4)


def test_deterministic_and_side_stream():
    inp = make_random_case(12, 3000, 1024, 64, 8, mask_frac=0.05)
    s = torch.cuda.Stream()
    a = run_case(inp.topk_idx, inp.x_bits, inp.topk_weights, 64, y_bits=inp.x_bits.repeat(8, 0))
    b = run_case(inp.topk_idx, inp.x_bits, inp.topk_weights, 64, y_bits=inp.x_bits.repeat(8, 0),
                 stream=s)
    for key in a:
        if a[key] is None or np.ndim(a[key]) == 0:
            assert a[key] == b[key], key
            continue
        np.testing.assert_array_equal(np.asarray(a[key]).view(np.uint8), np.asarray(b[key]).view(np.uint8))


def test_combine_non_finite_inputs():
    # expert rows holding +-inf and NaN: a sum with a NaN term, or with
    # infinities of both signs, is NaN on both sides (the NaN's sign and
    # payload are not compared); a sum with infinities of one sign is that
    # infinity; every other element is within the usual gate
    T, H, E, k = 96, 256, 8, 4
    inp = make_random_case(33, T, H, E, k, mask_frac=0.1)
    L = oracle.layout(inp.topk_idx, E)
    P = T * k
    rng = np.random.default_rng(34)
    y = make_gradient(P, H, 35)
    for bits, count in ((0x7F80, 60), (0xFF80, 60), (0x7FC1, 30), (0xFFC0, 30)):
        rows = rng.integers(0, max(L.n, 1), count)
        cols = rng.integers(0, H, count)
        y[rows, cols] = bits
    out = ep.ep_combine(x_dev(y), dev(L.slot), dev(inp.topk_weights), rows=P)
    torch.cuda.synchronize()
    got = float32_from_bf16_bits(bf16_bits(out)).astype(np.float64)
    ref_bits = oracle.combine(y, L.slot, inp.topk_weights)
    want = float32_from_bf16_bits(ref_bits).astype(np.float64)
    assert np.isnan(want).any() and np.isinf(want).any()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    inf = np.isinf(want)
    np.testing.assert_array_equal(got[inf], want[inf])
    fin = np.isfinite(want)
    tol = combine_tolerance(y, L.slot, inp.topk_weights, ref_bits)
    assert np.all(np.abs(got[fin] - want[fin]) <= tol[fin])


def test_combine_unit_weights_fp32_partial_overflow():
    # unit weights (the unweighted combine) over rows near the bf16 maximum:
    # the kernel accumulates in fp32 in slot order, so a partial sum past the
    # fp32 maximum becomes an infinity even where the exact sum is finite
    # (+m + m - m).  Checked against that fp32 accumulation written out in
    # numpy; the exact-sum oracle is compared where no partial sum overflows.
    T, H, k = 64, 128, 3
    m = 0x7F70  # bf16 3.19e38: two of them overflow fp32
    P = T * k
    slot = np.arange(P, dtype=np.int32).reshape(T, k)
    rng = np.random.default_rng(36)
    y = make_gradient(P, H, 37)
    pick = rng.random((T, H)) < 0.3
    for j, sign in ((0, 0), (1, 0), (2, 0x8000)):
        yj = y[j::k]
        yj[pick] = m | sign
    out = ep.ep_combine(x_dev(y), dev(slot), None, rows=P)
    torch.cuda.synchronize()
    got = bf16_bits(out)
    acc = np.zeros((T, H), np.float32)
    with np.errstate(over="ignore"):
        for j in range(k):
            acc = acc + float32_from_bf16_bits(y[j::k])    # fp32 adds, slot order
    u = acc.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)   # RNE (no NaN here)
    assert np.isinf(acc[pick]).all() and not np.isnan(acc).any()
    np.testing.assert_array_equal(got, want)
    ref = oracle.combine(y, slot, None)
    assert np.all(ref[pick] == m)                       # the exact sum is finite there
    tol = combine_tolerance(y, slot, None, ref)
    g64 = float32_from_bf16_bits(got).astype(np.float64)
    r64 = float32_from_bf16_bits(ref).astype(np.float64)
    assert np.all(np.abs(g64 - r64)[~pick] <= tol[~pick])
