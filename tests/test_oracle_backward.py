"""Pins for the oracle's backward passes, CPU only.

* combine backward: torch autograd in float64 (a library special case) gives
  the exact vector-Jacobian product of out = sum_j w * y[slot]; the oracle's
  grad_y must be that product rounded once to bf16 (checked by exhaustive
  table search in exact rationals) and its grad_w the float32 rounding of the
  exact dot products;
* dispatch backward: grad_x is the unit-weight reduction (exact rational
  brute force) and grad_w the gather of the row weight gradients (numpy
  fancy indexing);
* the adjoint identity <combine(y), g> = sum_r <y_r, grad_y_r>.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from combine_ep_layout_04_amd.inputs import (
    bf16_bits_from_float32, float32_from_bf16_bits, make_gradient, make_random_case,
)


def autograd_combine(y_bits, slot, w, g_bits):
    """Exact (float64) gradients of out = sum_j w[t,j] * y[slot[t,j]]."""
    T, k = slot.shape
    y = torch.tensor(float32_from_bf16_bits(y_bits), dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w if w is not None else np.ones((T, k), np.float32), dtype=torch.float64,
                      requires_grad=True)
    g = torch.tensor(float32_from_bf16_bits(g_bits), dtype=torch.float64)
    s = torch.tensor(slot.astype(np.int64))
    valid = (s >= 0).to(torch.float64)
    rows = y[s.clamp(min=0)] * valid[..., None]
    out = (wt[..., None] * rows).sum(dim=1)
    out.backward(g)
    return y.grad.numpy(), wt.grad.numpy()


@pytest.mark.parametrize("seed", range(6))
def test_combine_backward_vs_autograd(seed):
    T, H, E, k = 24, 40, 6, 3
    inp = make_random_case(100 + seed, T, H, E, k, mask_frac=0.25, dup_frac=1.0)
    L = oracle.layout(inp.topk_idx, E)
    rng = np.random.default_rng(seed)
    y = bf16_bits_from_float32((rng.standard_normal((T * k, H)) *
                                np.exp2(rng.integers(-6, 6, (T * k, H)))).astype(np.float32))
    g = make_gradient(T, H, seed)
    w = inp.topk_weights if seed % 2 else None
    gy, gw = oracle.combine_backward(g, y, L.slot, w)
    ref_gy, ref_gw = autograd_combine(y, L.slot, w, g)
    placed = np.zeros(T * k, bool)
    placed[L.slot[L.slot >= 0]] = True
    for r in np.nonzero(placed)[0]:
        for c in range(H):
            assert gy[r, c] == brute.bf16_round(Fraction(float(ref_gy[r, c]))), (r, c)
    assert not gy[~placed].any()
    np.testing.assert_array_equal(gw, ref_gw.astype(np.float32))
    assert np.all(gw[L.slot < 0] == 0)


def test_combine_backward_ties_round_to_even():
    # w * g exactly halfway between two bf16 values must round to the even one
    g = bf16_bits_from_float32(np.array([[1.0, 3.0, -1.0, 1.0 + 2 ** -7]], np.float32))
    w = np.array([[1.0 + 2 ** -8]], np.float32)      # 1 + 2^-8: the midpoint above 1
    slot = np.array([[0]], np.int32)
    gy, _ = oracle.combine_backward(g, None, slot, w)
    # 1*(1+2^-8): a tie between 1 and 1+2^-7 -> 1.0 (0x3F80), and -1.0
    # 3*(1+2^-8) = 3 + 0.75*2^-6 (bf16 spacing 2^-6 in [2,4)) -> 3 + 2^-6 (0x4041)
    # (1+2^-7)(1+2^-8) = 1 + 3*2^-8 + 2^-15: just above the midpoint -> 1 + 2^-6 (0x3F82)
    assert gy[0, 0] == 0x3F80 and gy[0, 2] == 0xBF80
    assert gy[0, 1] == 0x4041
    assert gy[0, 3] == 0x3F82


def tiny_product_case(seed=0):
    """Weights and gradients whose products land below 2^-116, around the
    bf16 subnormal range (2^-133 steps below 2^-126), with exact bf16
    midpoints among them, plus a NaN weight and a NaN-making 0 * inf."""
    rng = np.random.default_rng(seed)
    T, H, k = 6, 64, 2
    gexp = rng.integers(-110, -90, (T, H))
    g = bf16_bits_from_float32((rng.choice([-1.0, 1.0], (T, H)) * (1 + rng.integers(0, 128, (T, H)) / 128.0)
                                * np.exp2(gexp)).astype(np.float32))
    w = (rng.uniform(1, 2, (T, k)) * np.exp2(rng.integers(-40, -20, (T, k)))).astype(np.float32)
    # the counterexample to an fp32 product-error test: w * g = 1.25 * 2^-132
    # + 2^-155, a hair above a bf16 midpoint that fp32 cannot see
    w[0, 0] = np.float32(1.25 * 2.0 ** -32 + 2.0 ** -55)
    g[0, 0] = bf16_bits_from_float32(np.array([2.0 ** -100], np.float32))[0]
    # an exact midpoint below 2^-126: 1.5 * 2^-133 -> ties to even (2^-132)
    w[1, 0] = np.float32(1.5 * 2.0 ** -33)
    g[1, 0] = bf16_bits_from_float32(np.array([2.0 ** -100], np.float32))[0]
    w.view(np.uint32)[2, 1] = 0x7FFFFFFF           # a NaN whose high half is 0x7FFF
    g[3, 5] = 0x7F80                               # +inf gradient
    w[3, 0] = 0.0                                  # 0 * inf = NaN
    slot = np.arange(T * k, dtype=np.int32).reshape(T, k)
    return g, w, slot


def test_combine_backward_tiny_and_nan_products():
    g, w, slot = tiny_product_case()
    gy, _ = oracle.combine_backward(g, None, slot, w)
    T, k = slot.shape
    gf = float32_from_bf16_bits(g)
    for t in range(T):
        for j in range(k):
            r = slot[t, j]
            for c in range(g.shape[1]):
                wv, gv = float(w[t, j]), float(gf[t, c])
                if np.isnan(wv) or (wv == 0 and np.isinf(gv)):
                    assert gy[r, c] == 0x7FC0, (t, j, c)
                elif np.isinf(gv):
                    assert gy[r, c] == (0x7F80 if wv * gv > 0 else 0xFF80)
                else:
                    want = brute.bf16_round(Fraction(wv) * Fraction(gv))
                    if wv * gv < 0 or (wv * gv == 0 and np.signbit(wv) != np.signbit(gv)):
                        want |= 0x8000
                    assert gy[r, c] == want, (t, j, c)
    assert gy[0, 0] == 0x0003        # above the midpoint 2.5 * 2^-133
    assert gy[2, 0] == 0x0002        # the midpoint 1.5 * 2^-133 goes to even


def test_combine_backward_adjoint_identity():
    T, H, E, k = 64, 32, 8, 4
    inp = make_random_case(7, T, H, E, k, mask_frac=0.1)
    L = oracle.layout(inp.topk_idx, E)
    y = make_gradient(T * k, H, 11)
    g = make_gradient(T, H, 12)
    gy, gw = oracle.combine_backward(g, y, L.slot, inp.topk_weights)
    yf = float32_from_bf16_bits(y).astype(np.float64)
    # sum_t <out_t, g_t> with the exact (unrounded) out equals
    # sum_{t,j} w_tj * grad_w_tj and, up to the bf16 rounding of grad_y,
    # sum_r <y_r, grad_y_r>
    ref_gy, ref_gw = autograd_combine(y, L.slot, inp.topk_weights, g)
    lhs = float((inp.topk_weights.astype(np.float64) * ref_gw).sum())
    rhs_exact = float((yf * ref_gy).sum())
    assert abs(lhs - rhs_exact) <= 1e-9 * max(1.0, abs(lhs))
    rhs = float((yf * float32_from_bf16_bits(gy).astype(np.float64)).sum())
    assert abs(rhs - rhs_exact) <= 2.0 ** -8 * float(np.abs(yf * ref_gy).sum())
    lhs2 = float((inp.topk_weights.astype(np.float64) * gw.astype(np.float64)).sum())
    assert abs(lhs2 - lhs) <= 2.0 ** -23 * float(np.abs(inp.topk_weights * gw).sum()) + 1e-30


@pytest.mark.parametrize("seed", range(4))
def test_dispatch_backward(seed):
    T, H, E, k = 20, 24, 5, 3
    inp = make_random_case(200 + seed, T, H, E, k, mask_frac=0.3, dup_frac=1.0)
    L = oracle.layout(inp.topk_idx, E)
    rng = np.random.default_rng(seed)
    grad_recv = make_gradient(T * k, H, 300 + seed)
    grad_recv_w = rng.standard_normal(T * k).astype(np.float32)
    gx, gw = oracle.dispatch_backward(grad_recv, grad_recv_w, L.slot, T)
    np.testing.assert_array_equal(gx, brute.combine(grad_recv, L.slot, None))
    want = np.where(L.slot >= 0, grad_recv_w[np.maximum(L.slot, 0)], 0).astype(np.float32)
    np.testing.assert_array_equal(gw, want)
