"""CPU oracle for MoE token layout, dispatch and combine.

TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the CPU
baseline of the benchmark may import this package; the library under
``combine_ep_layout_04_amd`` never does, and this package imports nothing
from it.

``ep_oracle.c`` holds the plain C definitions (built with gcc by
:func:`build`, loaded with ctypes); :mod:`oracle.brute` holds pure-Python
brute force versions used to pin the C code on tiny inputs.  All functions
take and return numpy arrays:

* bf16 tensors travel as ``uint16`` bit patterns,
* ``topk_idx`` is int64 ``[T, k]`` with -1 for a masked slot,
* weights and scales are float32.

Which passage each function follows is stated next to its C definition.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")


def build(force: bool = True) -> str:
    """Compile ``ep_oracle.c`` into ``liboracle.so`` with gcc (single
    thread: the oracle), and the same source with -fopenmp into
    ``liboracle_omp.so`` (the multi-core CPU baseline)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    if force or not os.path.exists(_LIB_OMP):
        tmp = _LIB_OMP + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-fopenmp", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_OMP)
    return _LIB


_lib_omp: Optional[ctypes.CDLL] = None


def omp_lib() -> ctypes.CDLL:
    """The -fopenmp build: oracle_dispatch_bf16 and oracle_combine run their
    token loops on all host cores (the benchmark's multi-core baseline)."""
    global _lib_omp
    if _lib_omp is None:
        if not os.path.exists(_LIB_OMP):
            build(force=True)
        L = ctypes.CDLL(_LIB_OMP)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_dispatch_bf16.argtypes = [P, i64, i32, i32, P, P, P, P]
        L.oracle_dispatch_bf16.restype = None
        L.oracle_combine.argtypes = [P, P, P, i64, i32, i32, P]
        L.oracle_combine.restype = None
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = i32
        _lib_omp = L
    return _lib_omp


def dispatch_bf16_parallel(x_bits: np.ndarray, slot: np.ndarray, rows: Optional[int] = None) -> np.ndarray:
    """oracle_dispatch_bf16 on all host cores (no weights); [rows, H] uint16."""
    x = _c(x_bits, np.uint16)
    s = _c(slot, np.int32)
    T, H = x.shape
    k = s.shape[1]
    out = np.zeros((T * k if rows is None else int(rows), H), np.uint16)
    omp_lib().oracle_dispatch_bf16(_ptr(x), T, H, k, _ptr(s), None, _ptr(out), None)
    return out


def combine_parallel(y_bits: np.ndarray, slot: np.ndarray, topk_weights: Optional[np.ndarray]) -> np.ndarray:
    """oracle_combine on all host cores; [T, H] uint16."""
    y = _c(y_bits, np.uint16)
    s = _c(slot, np.int32)
    T, k = s.shape
    H = y.shape[1]
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    out = np.empty((T, H), np.uint16)
    omp_lib().oracle_combine(_ptr(y), _ptr(s), _ptr(w), T, H, k, _ptr(out))
    return out


def parallel_threads() -> int:
    return int(omp_lib().oracle_threads())


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e5m2_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e5m2_decode.restype = ctypes.c_double
        L.oracle_e5m2_encode.argtypes = [ctypes.c_float]
        L.oracle_e5m2_encode.restype = ctypes.c_uint8
        L.oracle_dispatch_quant.argtypes = [P, i64, i32, i32, P, P, i32, i32, P, P, P]
        L.oracle_dispatch_quant.restype = None
        L.oracle_dispatch_prequant.argtypes = [P, P, i64, i32, i32, P, P, P, P, P]
        L.oracle_dispatch_prequant.restype = None
        L.oracle_layout.argtypes = [P, i64, i32, i32, P, P, P, P, P]
        L.oracle_layout.restype = None
        L.oracle_layout_ex.argtypes = [P, i64, i32, i32, i32, i64, P, P, P, P, P, P]
        L.oracle_layout_ex.restype = None
        L.oracle_dispatch_bf16.argtypes = [P, i64, i32, i32, P, P, P, P]
        L.oracle_dispatch_bf16.restype = None
        L.oracle_dispatch_fp8.argtypes = [P, i64, i32, i32, P, P, P, P, P]
        L.oracle_dispatch_fp8.restype = None
        L.oracle_combine.argtypes = [P, P, P, i64, i32, i32, P]
        L.oracle_combine.restype = None
        L.oracle_combine_backward.argtypes = [P, P, P, P, i64, i32, i32, P, P]
        L.oracle_combine_backward.restype = None
        L.oracle_dispatch_backward.argtypes = [P, P, P, i64, i32, i32, P, P]
        L.oracle_dispatch_backward.restype = None
        L.oracle_routing_map.argtypes = [P, i64, i32, i32, P, P]
        L.oracle_routing_map.restype = None
        L.oracle_rank_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_rank_layout.restype = None
        L.oracle_dispatch_ranked.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P]
        L.oracle_dispatch_ranked.restype = None
        L.oracle_combine_ranked.argtypes = [P, P, i64, i32, i32, P]
        L.oracle_combine_ranked.restype = None
        L.oracle_dispatch_fused_permute.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, P,
                                                    P, P]
        L.oracle_dispatch_fused_permute.restype = None
        L.oracle_dispatch_fused_permute_prequant.argtypes = [P, P, P, P, i64, i32, i32, i32, i32,
                                                             i32, P, P, P, P, P, P]
        L.oracle_dispatch_fused_permute_prequant.restype = None
        L.oracle_dispatch_ranked_prequant.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, P, P, P,
                                                      P]
        L.oracle_dispatch_ranked_prequant.restype = None
        L.oracle_dispatch_ranked_backward.argtypes = [P, P, P, i64, P, P, i64, i32, i32, i32, i32,
                                                      P, P]
        L.oracle_dispatch_ranked_backward.restype = None
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ codecs --

def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(int(b) & 0xFFFF)


def bf16_from_double(d: float) -> int:
    return int(lib().oracle_bf16_from_double(float(d)))


def e4m3_decode(c: int) -> float:
    return lib().oracle_e4m3_decode(int(c) & 0xFF)


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def e5m2_decode(c: int) -> float:
    return lib().oracle_e5m2_decode(int(c) & 0xFF)


def e5m2_encode(v: float) -> int:
    return int(lib().oracle_e5m2_encode(float(v)))


# ------------------------------------------------------------------ layout --

class Layout:
    """Result of :func:`layout`: counts [E], offsets [E+1], slot [T,k],
    src [rows] (rows nothing maps to hold -1), and the invalid-index and
    dropped-pair counts."""

    def __init__(self, counts, offsets, slot, src, num_invalid, num_dropped=0):
        self.counts = counts
        self.offsets = offsets
        self.slot = slot
        self.src = src
        self.num_invalid = num_invalid
        self.num_dropped = num_dropped

    @property
    def n(self) -> int:
        """Rows of the layout (padding included): offsets[E]."""
        return int(self.offsets[-1])


def max_rows(T: int, k: int, E: int, alignment: int = 1, capacity: int = 0) -> int:
    """Rows a receive buffer needs for any routing of this shape."""
    if capacity > 0:
        return E * capacity
    return T * k + min(E, T * k) * (alignment - 1)


def layout(topk_idx: np.ndarray, num_experts: int, alignment: int = 1, capacity: int = 0) -> Layout:
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    E = int(num_experts)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    slot = np.zeros((T, k), np.int32)
    src = np.full(max(max_rows(T, k, E, alignment, capacity), T * k), -1, np.int32)
    bad = np.zeros(1, np.int32)
    dropped = np.zeros(1, np.int32)
    if alignment == 1 and capacity == 0:
        lib().oracle_layout(_ptr(idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(slot), _ptr(src),
                            _ptr(bad))
    else:
        lib().oracle_layout_ex(_ptr(idx), T, k, E, int(alignment), int(capacity), _ptr(counts),
                               _ptr(offsets), _ptr(slot), _ptr(src), _ptr(bad), _ptr(dropped))
    return Layout(counts, offsets, slot, src, int(bad[0]), int(dropped[0]))


# ---------------------------------------------------------------- dispatch --

def dispatch_bf16(x_bits: np.ndarray, slot: np.ndarray, topk_weights: Optional[np.ndarray] = None,
                  rows: Optional[int] = None):
    """Return (recv_x uint16 [rows, H], recv_w float32 [rows] or None).
    Rows nobody writes stay 0.  ``rows`` defaults to T*k."""
    x = _c(x_bits, np.uint16)
    s = _c(slot, np.int32)
    T, H = x.shape
    k = s.shape[1]
    R = T * k if rows is None else int(rows)
    if s.size and s.max() >= R:
        raise ValueError("a slot is beyond the receive buffer")
    recv = np.zeros((R, H), np.uint16)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rw = None if w is None else np.zeros(R, np.float32)
    lib().oracle_dispatch_bf16(_ptr(x), T, H, k, _ptr(s), _ptr(w), _ptr(recv), _ptr(rw))
    return recv, rw


def dispatch_fp8(x_bits: np.ndarray, slot: np.ndarray, topk_weights: Optional[np.ndarray] = None,
                 rows: Optional[int] = None):
    """Return (recv_q uint8 [rows, H], recv_scales float32 [rows, H/128],
    recv_w float32 [rows] or None)."""
    x = _c(x_bits, np.uint16)
    s = _c(slot, np.int32)
    T, H = x.shape
    if H % 128:
        raise ValueError("fp8 dispatch needs hidden % 128 == 0")
    k = s.shape[1]
    R = T * k if rows is None else int(rows)
    if s.size and s.max() >= R:
        raise ValueError("a slot is beyond the receive buffer")
    q = np.zeros((R, H), np.uint8)
    sc = np.zeros((R, H // 128), np.float32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rw = None if w is None else np.zeros(R, np.float32)
    lib().oracle_dispatch_fp8(_ptr(x), T, H, k, _ptr(s), _ptr(w), _ptr(q), _ptr(sc), _ptr(rw))
    return q, sc, rw


FORMATS = {"e4m3": 0, "e5m2": 1}
SCALE_MODES = {"fp32": 0, "pow2": 1, "ue8m0": 2}


def dispatch_quant(x_bits: np.ndarray, slot: np.ndarray, topk_weights: Optional[np.ndarray] = None,
                   fmt: str = "e4m3", scale: str = "fp32", rows: Optional[int] = None):
    """Return (recv_q uint8 [rows, H], recv_scales float32 or uint8
    [rows, H/128], recv_w float32 [rows] or None)."""
    x = _c(x_bits, np.uint16)
    s = _c(slot, np.int32)
    T, H = x.shape
    if H % 128:
        raise ValueError("fp8 dispatch needs hidden % 128 == 0")
    k = s.shape[1]
    R = T * k if rows is None else int(rows)
    if s.size and s.max() >= R:
        raise ValueError("a slot is beyond the receive buffer")
    q = np.zeros((R, H), np.uint8)
    sc = np.zeros((R, H // 128), np.uint8 if scale == "ue8m0" else np.float32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rw = None if w is None else np.zeros(R, np.float32)
    lib().oracle_dispatch_quant(_ptr(x), T, H, k, _ptr(s), _ptr(w), FORMATS[fmt], SCALE_MODES[scale],
                                _ptr(q), _ptr(sc), _ptr(rw))
    return q, sc, rw


def dispatch_prequant(xq: np.ndarray, xs: np.ndarray, slot: np.ndarray,
                      topk_weights: Optional[np.ndarray] = None, rows: Optional[int] = None):
    """Return (recv_q uint8 [rows, H], recv_scales float32 [rows, H/128],
    recv_w float32 [rows] or None) for pre-quantized input."""
    q_in = _c(xq, np.uint8)
    s_in = _c(xs, np.float32)
    s = _c(slot, np.int32)
    T, H = q_in.shape
    k = s.shape[1]
    R = T * k if rows is None else int(rows)
    if s.size and s.max() >= R:
        raise ValueError("a slot is beyond the receive buffer")
    q = np.zeros((R, H), np.uint8)
    sc = np.zeros((R, H // 128), np.float32)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    rw = None if w is None else np.zeros(R, np.float32)
    lib().oracle_dispatch_prequant(_ptr(q_in), _ptr(s_in), T, H, k, _ptr(s), _ptr(w), _ptr(q),
                                   _ptr(sc), _ptr(rw))
    return q, sc, rw


# ----------------------------------------------------------------- combine --

def combine(y_bits: np.ndarray, slot: np.ndarray, topk_weights: Optional[np.ndarray]) -> np.ndarray:
    """Return out uint16 [T, H] (bf16 bits)."""
    y = _c(y_bits, np.uint16)
    s = _c(slot, np.int32)
    T, k = s.shape
    H = y.shape[1]
    if s.size and s.max() >= y.shape[0]:
        raise ValueError("a slot is beyond the expert outputs")
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    out = np.zeros((T, H), np.uint16)
    lib().oracle_combine(_ptr(y), _ptr(s), _ptr(w), T, H, k, _ptr(out))
    return out


# ---------------------------------------------------------------- backward --

def combine_backward(g_bits: np.ndarray, y_bits: Optional[np.ndarray], slot: np.ndarray,
                     topk_weights: Optional[np.ndarray], rows: Optional[int] = None):
    """Return (grad_y uint16 [rows, H], grad_w float32 [T, k] or None).
    grad_w is computed when y is given.  Rows nothing maps to stay 0."""
    g = _c(g_bits, np.uint16)
    s = _c(slot, np.int32)
    T, H = g.shape
    k = s.shape[1]
    R = T * k if rows is None else int(rows)
    if s.size and s.max() >= R:
        raise ValueError("a slot is beyond the expert outputs")
    y = None if y_bits is None else _c(y_bits, np.uint16)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    gy = np.zeros((R, H), np.uint16)
    gw = None if y is None else np.zeros((T, k), np.float32)
    lib().oracle_combine_backward(_ptr(g), _ptr(y), _ptr(s), _ptr(w), T, H, k, _ptr(gy), _ptr(gw))
    return gy, gw


def dispatch_backward(grad_recv_bits: np.ndarray, grad_recv_w: Optional[np.ndarray],
                      slot: np.ndarray, T: int):
    """Return (grad_x uint16 [T, H], grad_w float32 [T, k] or None)."""
    gr = _c(grad_recv_bits, np.uint16)
    s = _c(slot, np.int32)
    k = s.shape[1]
    H = gr.shape[1]
    if s.size and s.max() >= gr.shape[0]:
        raise ValueError("a slot is beyond the row gradients")
    grw = None if grad_recv_w is None else _c(grad_recv_w, np.float32)
    gx = np.zeros((T, H), np.uint16)
    gw = None if grw is None else np.zeros((T, k), np.float32)
    lib().oracle_dispatch_backward(_ptr(gr), _ptr(grw), _ptr(s), T, H, k, _ptr(gx), _ptr(gw))
    return gx, gw


# ------------------------------------------------ per-(token, rank) path --

def routing_map(topk_idx: np.ndarray, num_experts: int):
    """Return (map uint8 [T, ceil(E/8)], num_invalid): bit e % 8 of byte
    e // 8 of row t is set iff token t selects expert e."""
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    E = int(num_experts)
    m = np.zeros((T, (E + 7) // 8), np.uint8)
    bad = np.zeros(1, np.int32)
    lib().oracle_routing_map(_ptr(idx), T, k, E, _ptr(m), _ptr(bad))
    return m, int(bad[0])


class RankLayout:
    """Result of :func:`rank_layout` for one rank: sparse_to_dense [T, G],
    local_map uint8 [G*T, E/G], recv_src [G*T], recv_topk_idx [G*T, k_out],
    expert_counts [E/G], num_recv, num_overflow."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def rank_layout(global_map: np.ndarray, T: int, E: int, G: int, rank: int, k_out: int) -> RankLayout:
    m = _c(global_map, np.uint8)
    if m.shape != (G * T, (E + 7) // 8) or E % G or not 0 <= rank < G:
        raise ValueError("bad rank layout shape")
    El = E // G
    R = G * T
    s2d = np.zeros((T, G), np.int32)
    lm = np.zeros((R, El), np.uint8)
    src = np.zeros(R, np.int32)
    rti = np.zeros((R, k_out), np.int64)
    cnt = np.zeros(El, np.int32)
    nr = np.zeros(1, np.int32)
    ov = np.zeros(1, np.int32)
    lib().oracle_rank_layout(_ptr(m), T, E, G, rank, k_out, _ptr(s2d), _ptr(lm), _ptr(src),
                             _ptr(rti), _ptr(cnt), _ptr(nr), _ptr(ov))
    return RankLayout(sparse_to_dense=s2d, local_map=lm, recv_src=src, recv_topk_idx=rti,
                      expert_counts=cnt, num_recv=int(nr[0]), num_overflow=int(ov[0]))


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[None if a is None else a.ctypes.data for a in arrs])


def dispatch_ranked(x_bits: np.ndarray, topk_idx: np.ndarray, topk_weights: Optional[np.ndarray],
                    E: int, G: int, sparse_to_dense: np.ndarray, rows, with_weights: bool = True):
    """Return (dest_x list of G uint16 [rows_d, H], dest_w list of G float32
    [rows_d, k] or None).  ``rows`` is one int or G ints; unwritten rows
    stay 0."""
    x = _c(x_bits, np.uint16)
    idx = _c(topk_idx, np.int64)
    s2d = _c(sparse_to_dense, np.int32)
    T, H = x.shape
    k = idx.shape[1]
    rows = [int(rows)] * G if np.isscalar(rows) else [int(r) for r in rows]
    for d in range(G):
        if s2d.size and s2d[:, d].max() >= rows[d]:
            raise ValueError("a row is beyond a destination buffer")
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    dx = [np.zeros((rows[d], H), np.uint16) for d in range(G)]
    dw = [np.zeros((rows[d], k), np.float32) for d in range(G)] if with_weights else None
    lib().oracle_dispatch_ranked(_ptr(x), _ptr(idx), _ptr(w), T, H, k, int(E), G, _ptr(s2d),
                                 _ptr_array(dx), None if dw is None else _ptr_array(dw))
    return dx, dw


def combine_ranked(src_y, sparse_to_dense: np.ndarray) -> np.ndarray:
    """Return out uint16 [T, H]: the fp64 sum over ranks, rounded once."""
    ys = [_c(y, np.uint16) for y in src_y]
    s2d = _c(sparse_to_dense, np.int32)
    T, G = s2d.shape
    if len(ys) != G:
        raise ValueError("one source buffer per rank")
    H = ys[0].shape[1]
    for d in range(G):
        if s2d.size and s2d[:, d].max() >= ys[d].shape[0]:
            raise ValueError("a row is beyond a source buffer")
    out = np.zeros((T, H), np.uint16)
    lib().oracle_combine_ranked(_ptr_array(ys), _ptr(s2d), T, H, G, _ptr(out))
    return out


def dispatch_ranked_backward(grad_recv_x, grad_recv_w, recv_topk_idx, topk_idx: np.ndarray,
                             sparse_to_dense: np.ndarray, E: int):
    """Backward of the once-per-rank dispatch for one sending rank.
    ``grad_recv_x`` / ``grad_recv_w`` / ``recv_topk_idx``: lists of the G
    receivers' row gradients (uint16 [rows, H], or None for no grad_x),
    weight gradients (float32 [rows, k], or None for no grad_w) and listed
    local experts (int64 [rows, k], from rank_layout with k_out = k).
    Returns (grad_x uint16 [T, H] or None, grad_w float32 [T, k] or None)."""
    idx = _c(topk_idx, np.int64)
    s2d = _c(sparse_to_dense, np.int32)
    T, k = idx.shape
    G = s2d.shape[1]
    if E % G:
        raise ValueError("E must be a multiple of G")
    rti = [_c(r, np.int64) for r in recv_topk_idx]
    rows = rti[0].shape[0]
    if len(rti) != G or any(r.shape != (rows, k) for r in rti):
        raise ValueError("one [rows, k] recv_topk_idx per rank")
    gx = gw = None
    gxs = gws = None
    H = 0
    if grad_recv_x is not None:
        gxs = [_c(g, np.uint16) for g in grad_recv_x]
        H = gxs[0].shape[1]
        for d in range(G):
            if gxs[d].shape[0] != rows or (s2d.size and s2d[:, d].max() >= rows):
                raise ValueError("row gradients must have the receive rows")
        gx = np.zeros((T, H), np.uint16)
    if grad_recv_w is not None:
        gws = [_c(g, np.float32) for g in grad_recv_w]
        if any(g.shape != (rows, k) for g in gws):
            raise ValueError("weight gradients must be [rows, k]")
        gw = np.zeros((T, k), np.float32)
    lib().oracle_dispatch_ranked_backward(
        None if gxs is None else _ptr_array(gxs), None if gws is None else _ptr_array(gws),
        _ptr_array(rti), rows, _ptr(idx), _ptr(s2d), T, H, k, int(E), G, _ptr(gx), _ptr(gw))
    return gx, gw


def dispatch_fused_permute(src_x, src_idx, src_w, E: int, rank: int, recv_src: np.ndarray,
                           recv_topk_idx: np.ndarray, slot: np.ndarray, rows: int,
                           with_weights: bool = True):
    """Receiver-side dispatch with the permute fused in.  ``src_x`` /
    ``src_idx`` / ``src_w`` are lists of the G ranks' tokens (uint16 [T, H]),
    topk_idx (int64 [T, k]) and weights (float32 [T, k] or None).  Returns
    (recv_x uint16 [rows, H], recv_w float32 [rows] or None); unwritten rows
    stay 0."""
    G = len(src_x)
    xs = [_c(x, np.uint16) for x in src_x]
    ids = [_c(i, np.int64) for i in src_idx]
    ws = [None if w is None else _c(w, np.float32) for w in src_w]
    T, H = xs[0].shape
    k = ids[0].shape[1]
    rs = _c(recv_src, np.int32)
    rti = _c(recv_topk_idx, np.int64)
    sl = _c(slot, np.int32)
    if rs.shape != (G * T,) or rti.shape != (G * T, k) or sl.shape != (G * T, k):
        raise ValueError("receive-side arrays must have G*T rows and k columns")
    if sl.size and sl.max() >= rows:
        raise ValueError("a slot is beyond the receive buffer")
    out = np.zeros((rows, H), np.uint16)
    rw = np.zeros(rows, np.float32) if with_weights else None
    wtab = None if all(w is None for w in ws) else _ptr_array(ws)
    lib().oracle_dispatch_fused_permute(_ptr_array(xs), _ptr_array(ids), wtab, T, H, k, int(E), G,
                                        int(rank), _ptr(rs), _ptr(rti), _ptr(sl), _ptr(out),
                                        _ptr(rw))
    return out, rw


def dispatch_fused_permute_prequant(src_q, src_s, src_idx, src_w, E: int, rank: int,
                                    recv_src: np.ndarray, recv_topk_idx: np.ndarray,
                                    slot: np.ndarray, rows: int, with_weights: bool = True):
    """oracle_dispatch_fused_permute for tokens already cast to 8 bits:
    ``src_q`` / ``src_s`` are lists of the G ranks' code rows (uint8 [T, H])
    and scale rows (float32 [T, H/128]).  Returns (recv_q uint8 [rows, H],
    recv_s float32 [rows, H/128], recv_w float32 [rows] or None); unwritten
    rows stay 0."""
    G = len(src_q)
    qs = [_c(q, np.uint8) for q in src_q]
    ss = [_c(x, np.float32) for x in src_s]
    ids = [_c(i, np.int64) for i in src_idx]
    ws = [None if w is None else _c(w, np.float32) for w in src_w]
    T, H = qs[0].shape
    nb = H // 128
    k = ids[0].shape[1]
    rs = _c(recv_src, np.int32)
    rti = _c(recv_topk_idx, np.int64)
    sl = _c(slot, np.int32)
    if rs.shape != (G * T,) or rti.shape != (G * T, k) or sl.shape != (G * T, k):
        raise ValueError("receive-side arrays must have G*T rows and k columns")
    if sl.size and sl.max() >= rows:
        raise ValueError("a slot is beyond the receive buffer")
    if any(x.shape != (T, nb) for x in ss):
        raise ValueError("every src_s must be [T, H/128]")
    out_q = np.zeros((rows, H), np.uint8)
    out_s = np.zeros((rows, nb), np.float32)
    rw = np.zeros(rows, np.float32) if with_weights else None
    wtab = None if all(w is None for w in ws) else _ptr_array(ws)
    lib().oracle_dispatch_fused_permute_prequant(_ptr_array(qs), _ptr_array(ss), _ptr_array(ids),
                                                 wtab, T, H, k, int(E), G, int(rank), _ptr(rs),
                                                 _ptr(rti), _ptr(sl), _ptr(out_q), _ptr(out_s),
                                                 _ptr(rw))
    return out_q, out_s, rw


def dispatch_ranked_prequant(xq: np.ndarray, xs: np.ndarray, topk_idx: np.ndarray,
                             topk_weights: Optional[np.ndarray], E: int, G: int,
                             sparse_to_dense: np.ndarray, rows, with_weights: bool = True):
    """Once-per-rank dispatch of pre-quantized tokens: returns (dest_q list of
    G uint8 [rows_d, H], dest_s list of G float32 [rows_d, H/128], dest_w
    list of G float32 [rows_d, k] or None)."""
    q = _c(xq, np.uint8)
    sc = _c(xs, np.float32)
    idx = _c(topk_idx, np.int64)
    s2d = _c(sparse_to_dense, np.int32)
    T, H = q.shape
    k = idx.shape[1]
    nb = H // 128
    rows = [int(rows)] * G if np.isscalar(rows) else [int(r) for r in rows]
    for d in range(G):
        if s2d.size and s2d[:, d].max() >= rows[d]:
            raise ValueError("a row is beyond a destination buffer")
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    dq = [np.zeros((rows[d], H), np.uint8) for d in range(G)]
    ds = [np.zeros((rows[d], nb), np.float32) for d in range(G)]
    dw = [np.zeros((rows[d], k), np.float32) for d in range(G)] if with_weights else None
    lib().oracle_dispatch_ranked_prequant(_ptr(q), _ptr(sc), _ptr(idx), _ptr(w), T, H, k, int(E),
                                          G, _ptr(s2d), _ptr_array(dq), _ptr_array(ds),
                                          None if dw is None else _ptr_array(dw))
    return dq, ds, dw


def dispatch_ranked_quant(x_bits: np.ndarray, topk_idx: np.ndarray,
                          topk_weights: Optional[np.ndarray], E: int, G: int,
                          sparse_to_dense: np.ndarray, rows, fmt: str = "e4m3",
                          scale: str = "fp32", with_weights: bool = True):
    """The 8-bit cast sent once per rank (NCCL EP page, ncclEpDispatch: fp8
    output with per-128-channel scales, and its high-throughput branch, one
    copy per rank), by its definition: each token cast once as
    oracle_dispatch_quant casts it, then its code and scale rows sent by
    oracle_dispatch_ranked_prequant.  UE8M0 scale bytes travel through that
    copy as the fp32 values 0..255, which it moves unchanged.  Returns
    (dest_q list of G uint8 [rows_d, H], dest_s list of G [rows_d, H/128]
    float32 or uint8, dest_w list of G float32 [rows_d, k] or None)."""
    x = _c(x_bits, np.uint16)
    T = x.shape[0]
    q_tok, s_tok, _ = dispatch_quant(x, np.arange(T, dtype=np.int32)[:, None], fmt=fmt,
                                     scale=scale)
    dq, ds, dw = dispatch_ranked_prequant(q_tok, s_tok.astype(np.float32), topk_idx,
                                          topk_weights, E, G, sparse_to_dense, rows,
                                          with_weights)
    if scale == "ue8m0":
        ds = [v.astype(np.uint8) for v in ds]
    return dq, ds, dw
