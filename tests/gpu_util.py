"""Helpers for the GPU parity tests: host <-> device copies of the seeded
inputs and the bf16 one-ulp comparison."""

import numpy as np
import torch

DEV = "cuda:0"


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def x_dev(x_bits: np.ndarray) -> torch.Tensor:
    return dev(x_bits.view(np.int16), torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 at |v| (2^-133 below the normal range)."""
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def check_within_one_ulp(got_bits: np.ndarray, ref_bits: np.ndarray, what: str):
    """|got - ref| <= one bf16 ulp of ref, elementwise; returns the max
    relative error max|got-ref| / max(|ref|, 2^-126)."""
    g = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = (ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    diff = np.abs(g - r)
    bad = diff > bf16_ulp(r)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond 1 bf16 ulp, first at "
                             f"{tuple(i)}: got {g[tuple(i)]!r} want {r[tuple(i)]!r}")
    rel = diff / np.maximum(np.abs(r), 2.0 ** -126)
    return float(rel.max()) if rel.size else 0.0
