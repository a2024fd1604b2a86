"""Seeded synthetic inputs for MoE token dispatch / combine.

This module only draws random inputs and builds the stand-in expert outputs
that a test feeds to combine.  It contains none of the layout, dispatch or
combine arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
can consume exactly the same bytes.

Workload shapes follow the examples on the DeepEP API page ("MoE Dispatch and
Combine for Training/Inference with ElasticBuffer", "dispatch()" example:
x [8192, 7168] bf16, 256 experts, top-8, fp32 weights) and the NeMo fused_a2a
page (``HybridEPDispatch``: ``topk_idx`` uses -1 for unused slots).

Every array is produced from ``numpy.random.default_rng(seed)`` in a fixed
draw order:

1. x ~ N(0, 1) as float32 ``[T, H]``; for outlier workloads a fixed fraction of
   rows (chosen without replacement) is multiplied by a factor in float32;
   then rounded to bf16 (round-to-nearest-even, done by torch on the CPU).
2. routing ``topk_idx`` int64 ``[T, k]``:
   * ``uniform``: the first k columns of ``argsort(U[T, E])`` -- a uniformly
     random k-subset of distinct experts per row, in random order;
   * ``zipf``: a seeded expert permutation gives popularity p(perm[r-1]) ~
     r^-s; each row draws k distinct experts by Gumbel-top-k over log p;
   * then a fixed fraction of the T*k flat slots, chosen without
     replacement, is set to -1 (masked).
3. weights: u ~ U(0, 1) float32 ``[T, k]``, zero where masked, divided by the
   row sum in float32 (an all-masked row keeps zero weights).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "Inputs",
    "make_inputs",
    "make_random_case",
    "bf16_bits_from_float32",
    "float32_from_bf16_bits",
    "expert_ids_of_rows",
    "expert_outputs_scaled",
    "expert_outputs_dequant",
    "make_gradient",
    "make_routing",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    routing: str = "uniform"          # "uniform" | "zipf"
    zipf_s: float = 1.2
    mask_frac: float = 0.0
    outlier_frac: float = 0.0
    outlier_scale: float = 100.0
    fp8: bool = False                  # dispatch casts to e4m3 with per-128 scales
    expert: str = "identity"           # stand-in expert used before combine
    seed: int = 0

    @property
    def pairs(self) -> int:
        return self.T * self.k


# The five seeded workloads.  "headline" is the throughput workload.
WORKLOADS = {
    "tiny": Workload("tiny", T=128, H=256, E=8, k=2),
    "mid": Workload("mid", T=4096, H=2048, E=64, k=4, expert="scaled"),
    "headline": Workload("headline", T=8192, H=7168, E=256, k=8),
    "skewed": Workload("skewed", T=8192, H=7168, E=256, k=8, routing="zipf",
                       zipf_s=1.2, mask_frac=0.05),
    "fp8": Workload("fp8", T=8192, H=7168, E=256, k=8, outlier_frac=0.01,
                    outlier_scale=100.0, fp8=True, expert="dequant"),
}


@dataclasses.dataclass
class Inputs:
    workload: Workload
    x_bits: np.ndarray        # uint16 [T, H], bf16 bit patterns
    topk_idx: np.ndarray      # int64  [T, k], -1 = masked
    topk_weights: np.ndarray  # float32 [T, k]


def bf16_bits_from_float32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) with torch's CPU RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def float32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _route_uniform(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int64)


def _route_zipf(rng: np.random.Generator, T: int, E: int, k: int, s: float) -> np.ndarray:
    perm = rng.permutation(E)
    p = np.empty(E, dtype=np.float64)
    p[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    g = rng.gumbel(size=(T, E))
    scores = np.log(p)[None, :] + g
    return np.argsort(-scores, axis=1, kind="stable")[:, :k].astype(np.int64)


def _weights(rng: np.random.Generator, idx: np.ndarray) -> np.ndarray:
    u = rng.random(idx.shape, dtype=np.float32)
    u[idx < 0] = 0.0
    s = u.sum(axis=1, dtype=np.float32, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        w = np.where(s > 0, u / np.where(s > 0, s, np.float32(1)), np.float32(0))
    return w.astype(np.float32)


def make_inputs(w: Workload, T: Optional[int] = None) -> Inputs:
    """Draw the seeded inputs of workload ``w`` (optionally with fewer tokens).

    With ``T`` smaller than ``w.T`` the same recipe is run at that size (a
    different draw, not a prefix of the full one).
    """
    T = w.T if T is None else int(T)
    rng = np.random.default_rng(w.seed)
    x = rng.standard_normal((T, w.H), dtype=np.float32)
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * T))
        rows = rng.choice(T, size=n_out, replace=False)
        x[rows] *= np.float32(w.outlier_scale)
    if w.routing == "uniform":
        idx = _route_uniform(rng, T, w.E, w.k)
    elif w.routing == "zipf":
        idx = _route_zipf(rng, T, w.E, w.k, w.zipf_s)
    else:
        raise ValueError(f"unknown routing {w.routing!r}")
    if w.mask_frac > 0:
        n_mask = int(round(w.mask_frac * T * w.k))
        flat = rng.choice(T * w.k, size=n_mask, replace=False)
        idx.reshape(-1)[flat] = -1
    wts = _weights(rng, idx)
    return Inputs(w, bf16_bits_from_float32(x), np.ascontiguousarray(idx), wts)


def make_random_case(seed: int, T: int, H: int, E: int, k: int,
                     mask_frac: float = 0.0, dup_frac: float = 0.0,
                     invalid_frac: float = 0.0) -> Inputs:
    """Small adversarial routing: independent draws per slot (duplicates
    allowed), some slots masked (-1) and some out of range (>= E or < -1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H), dtype=np.float32)
    if dup_frac > 0:
        idx = rng.integers(0, E, size=(T, k), dtype=np.int64)
    else:
        idx = _route_uniform(rng, T, E, k) if k <= E else rng.integers(0, E, size=(T, k), dtype=np.int64)
    m = rng.random((T, k)) < mask_frac
    idx[m] = -1
    bad = rng.random((T, k)) < invalid_frac
    if bad.any():
        # out of range, including values whose low 32 bits read as a valid
        # expert (1 << 40, 2^32 + 5, INT64_MIN) or as the mask (-1:
        # 2^32 - 1, INT64_MAX) if an index were narrowed before the check
        i64 = np.iinfo(np.int64)
        choices = np.array([E, E + 3, -2, -7, 1 << 40, -(1 << 40), (1 << 32) - 1, (1 << 32) + 5,
                            i64.max, i64.min], dtype=np.int64)
        idx[bad] = choices[rng.integers(0, len(choices), size=int(bad.sum()))]
    wts = _weights(rng, np.where((idx >= 0) & (idx < E), idx, -1))
    wl = Workload("random", T=T, H=H, E=E, k=k, seed=seed)
    return Inputs(wl, bf16_bits_from_float32(x), np.ascontiguousarray(idx), wts)


def expert_ids_of_rows(offsets: np.ndarray, n_rows: int) -> np.ndarray:
    """Expert id of each received row r < offsets[-1], from exclusive offsets."""
    off = np.asarray(offsets, dtype=np.int64)
    counts = np.diff(off)
    e = np.repeat(np.arange(len(counts), dtype=np.int64), counts)
    out = np.full(n_rows, -1, dtype=np.int64)
    out[: len(e)] = e
    return out


def expert_outputs_scaled(recv_bits: np.ndarray, offsets: np.ndarray, denom: float = 64.0) -> np.ndarray:
    """Stand-in expert: row r of expert e becomes bf16(row * (e+1)/denom).

    The product of a bf16 value and (e+1)/64 is exact in float32 for e < 64,
    so torch's float32 -> bf16 cast is the only rounding.  Rows past the last
    received row are left zero.
    """
    n = int(offsets[-1])
    e = expert_ids_of_rows(offsets, recv_bits.shape[0])
    f = float32_from_bf16_bits(recv_bits[:n]).astype(np.float32)
    scale = ((e[:n] + 1).astype(np.float32) / np.float32(denom))[:, None]
    y = np.zeros_like(recv_bits)
    y[:n] = bf16_bits_from_float32(f * scale)
    return y


def expert_outputs_dequant(q: np.ndarray, scales: np.ndarray, n: int) -> np.ndarray:
    """Stand-in expert after an fp8 dispatch: bf16(decode_e4m3(q) * scale).

    Uses torch's float8_e4m3fn -> float32 widening (exact) and torch's
    float32 -> bf16 cast.  Rows >= n are zero.
    """
    R, H = q.shape
    nb = H // 128
    y = np.zeros((R, H), dtype=np.uint16)
    if n == 0:
        return y
    qt = torch.from_numpy(np.ascontiguousarray(q[:n])).view(torch.float8_e4m3fn).to(torch.float32)
    st = torch.from_numpy(np.ascontiguousarray(scales[:n], dtype=np.float32))
    prod = (qt.view(n, nb, 128) * st.view(n, nb, 1)).view(n, H)
    y[:n] = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return y


def make_gradient(rows: int, H: int, seed: int = 1) -> np.ndarray:
    """A seeded upstream gradient: N(0,1) float32 [rows, H] rounded to bf16."""
    rng = np.random.default_rng(seed)
    return bf16_bits_from_float32(rng.standard_normal((rows, H), dtype=np.float32))


def make_routing(T: int, E: int, k: int, seed: int) -> np.ndarray:
    """Uniform routing alone: int64 [T, k], a uniformly random k-subset of
    distinct experts per token (the ``uniform`` recipe above, drawn from
    ``default_rng(seed)`` with no token rows), for the other ranks of a
    simulated multi-rank map."""
    return np.ascontiguousarray(_route_uniform(np.random.default_rng(seed), T, E, k))
