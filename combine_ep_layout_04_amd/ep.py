"""Python binding of libep.so (the C ABI in include/ep.h).

Argument marshalling only: every step of layout, dispatch and combine runs
in the HIP kernels behind the C ABI.  PyTorch provides device memory and
the stream.  There is no fallback: if the library is missing or a call
fails, an exception is raised.

Two levels, with the C names:

* ``lib()`` returns the raw ``ctypes`` handle whose functions take integer
  device addresses (``tensor.data_ptr()``) and a stream handle;
* ``ep_layout``, ``ep_dispatch``, ``ep_combine`` take torch tensors, check
  dtype / shape / device, allocate outputs with torch when not given, and
  launch on ``stream`` (default: torch's current stream).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep.so")

EP_SUCCESS = 0
EP_INVALID_ARGUMENT = 1
EP_UNSUPPORTED = 2
EP_RUNTIME_ERROR = 3
EP_OUT_BF16 = 0
EP_OUT_FP8_E4M3 = 1
EP_OUT_FP8_E5M2 = 2
EP_SCALE_FP32 = 0
EP_SCALE_FP32_POW2 = 1
EP_SCALE_UE8M0 = 2
_FORMATS = {"e4m3": EP_OUT_FP8_E4M3, "e5m2": EP_OUT_FP8_E5M2}
_SCALES = {"fp32": EP_SCALE_FP32, "pow2": EP_SCALE_FP32_POW2, "ue8m0": EP_SCALE_UE8M0}
EP_MAX_EXPERTS = 1024
EP_MAX_TOPK = 64
EP_MAX_HIDDEN = 65536
EP_MAX_ALIGNMENT = 4096
EP_MAX_RANKS = 64

# every symbol include/ep.h declares
SYMBOLS = ("ep_version", "ep_status_string", "ep_last_error", "ep_layout_workspace_size",
           "ep_layout", "ep_layout_noalloc", "ep_layout_ex", "ep_layout_max_rows", "ep_dispatch", "ep_dispatch_ex",
           "ep_dispatch_prequantized", "ep_combine",
           "ep_combine_backward", "ep_dispatch_backward", "ep_routing_map",
           "ep_rank_layout_workspace_size", "ep_rank_layout", "ep_dispatch_ranked",
           "ep_dispatch_ranked_prequantized", "ep_dispatch_ranked_fp8", "ep_dispatch_fused_permute",
           "ep_dispatch_fused_permute_prequantized", "ep_combine_ranked",
           "ep_dispatch_ranked_backward", "ep_dispatch_colmajor_workspace_size",
           "ep_dispatch_colmajor_scales", "ep_dispatch_prequantized_colmajor")


class EpError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {message}")


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libep.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m combine_ep_layout_04_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.ep_version.argtypes = []
        L.ep_version.restype = i32
        L.ep_status_string.argtypes = [i32]
        L.ep_status_string.restype = ctypes.c_char_p
        L.ep_last_error.argtypes = []
        L.ep_last_error.restype = ctypes.c_char_p
        L.ep_layout_workspace_size.argtypes = [i64, i32, i32]
        L.ep_layout_workspace_size.restype = sz
        L.ep_layout.argtypes = [P, i64, i32, i32, P, P, P, P, P, P, sz, P]
        L.ep_layout.restype = i32
        L.ep_layout_noalloc.argtypes = [P, i64, i32, i32, P, P, P, P, P, P]
        L.ep_layout_noalloc.restype = i32
        L.ep_layout_ex.argtypes = [P, i64, i32, i32, i32, i64, P, P, P, P, P, P, P, sz, P]
        L.ep_layout_ex.restype = i32
        L.ep_layout_max_rows.argtypes = [i64, i32, i32, i32, i64]
        L.ep_layout_max_rows.restype = i64
        L.ep_dispatch.argtypes = [P, i64, i32, i32, P, P, i32, P, P, P, P]
        L.ep_dispatch.restype = i32
        L.ep_dispatch_ex.argtypes = [P, i64, i32, i32, P, P, i32, i32, P, P, P, i64, P]
        L.ep_dispatch_ex.restype = i32
        L.ep_dispatch_colmajor_workspace_size.argtypes = [i64, i32, i32]
        L.ep_dispatch_colmajor_workspace_size.restype = sz
        L.ep_dispatch_colmajor_scales.argtypes = [P, i64, i32, i32, P, P, P, i32, i32, P, P, P, i64,
                                                  i64, P, sz, P]
        L.ep_dispatch_colmajor_scales.restype = i32
        L.ep_dispatch_prequantized.argtypes = [P, P, i64, i32, i32, P, P, P, P, P, i64, P]
        L.ep_dispatch_prequantized.restype = i32
        L.ep_dispatch_prequantized_colmajor.argtypes = [P, P, i64, i32, i32, P, P, P, P, P, P, i64,
                                                        i64, P]
        L.ep_dispatch_prequantized_colmajor.restype = i32
        L.ep_combine.argtypes = [P, P, P, i64, i32, i32, P, P]
        L.ep_combine.restype = i32
        L.ep_combine_backward.argtypes = [P, P, P, P, i64, i32, i32, P, P, P]
        L.ep_combine_backward.restype = i32
        L.ep_dispatch_backward.argtypes = [P, P, P, i64, i32, i32, P, P, P]
        L.ep_dispatch_backward.restype = i32
        L.ep_routing_map.argtypes = [P, i64, i32, i32, P, P, P]
        L.ep_routing_map.restype = i32
        L.ep_rank_layout_workspace_size.argtypes = [i64, i32, i32]
        L.ep_rank_layout_workspace_size.restype = sz
        L.ep_rank_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, sz, P]
        L.ep_rank_layout.restype = i32
        L.ep_dispatch_ranked.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, i64, P]
        L.ep_dispatch_ranked.restype = i32
        L.ep_dispatch_ranked_prequantized.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, P, P, P,
                                                      P, i64, P]
        L.ep_dispatch_ranked_prequantized.restype = i32
        L.ep_dispatch_ranked_fp8.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, i32, i32, P, P,
                                             P, i64, P]
        L.ep_dispatch_ranked_fp8.restype = i32
        L.ep_dispatch_fused_permute.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P,
                                                i64, P, P, P]
        L.ep_dispatch_fused_permute.restype = i32
        L.ep_dispatch_fused_permute_prequantized.argtypes = [P, P, P, P, i64, i32, i32, i32, i32,
                                                             i32, P, P, P, P, i64, P, P, P, P]
        L.ep_dispatch_fused_permute_prequantized.restype = i32
        L.ep_combine_ranked.argtypes = [P, i64, P, i64, i32, i32, P, P]
        L.ep_combine_ranked.restype = i32
        L.ep_dispatch_ranked_backward.argtypes = [P, P, i64, P, P, i64, i32, i32, i32, i32, P, P,
                                                  P]
        L.ep_dispatch_ranked_backward.restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ep_status_string(int(status)).decode()


def last_error() -> str:
    return lib().ep_last_error().decode()


def version() -> int:
    return int(lib().ep_version())


def layout_workspace_size(num_tokens: int, num_topk: int, num_experts: int) -> int:
    return int(lib().ep_layout_workspace_size(int(num_tokens), int(num_topk), int(num_experts)))


def layout_max_rows(num_tokens: int, num_topk: int, num_experts: int, alignment: int = 1,
                    capacity: int = 0) -> int:
    """Rows a receive buffer needs for any routing of this shape (-1 if the
    arguments are invalid)."""
    return int(lib().ep_layout_max_rows(int(num_tokens), int(num_topk), int(num_experts),
                                        int(alignment), int(capacity)))


def _check(status: int, where: str) -> None:
    if status != EP_SUCCESS:
        raise EpError(status, where, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, numel: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")


# ------------------------------------------------------------------ layout --

def ep_layout(topk_idx: torch.Tensor, num_experts: int, *, alignment: int = 1, capacity: int = 0,
              counts=None, offsets=None, slot=None, src=None, num_invalid=None,
              num_dropped=None, workspace=None, want_src: bool = True,
              want_invalid: bool = True, stream=None):
    """Routing layout of ``topk_idx`` (int64 [T, k], -1 = masked).

    ``alignment`` / ``capacity`` select ep_layout_ex's segment placement
    (packed segments starting on multiples of ``alignment``, or a fixed
    ``capacity`` rows per expert with overflow dropped).

    Returns (counts int32 [E], offsets int32 [E+1], slot int32 [T, k],
    src int32 [rows] or None, num_invalid int32 [1] or None); with a
    capacity, ``num_dropped`` (int32 [1]) is filled when given.  ``rows`` is
    layout_max_rows(...).
    """
    _need(topk_idx, "topk_idx", torch.int64)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be 2-D [num_tokens, num_topk]")
    T, k = topk_idx.shape
    E = int(num_experts)
    rows = layout_max_rows(T, k, E, alignment, capacity)
    if rows < 0:
        raise ValueError("invalid layout shape, alignment or capacity")
    dev = topk_idx.device
    i32 = dict(dtype=torch.int32, device=dev)
    counts = torch.empty(E, **i32) if counts is None else counts
    offsets = torch.empty(E + 1, **i32) if offsets is None else offsets
    slot = torch.empty((T, k), **i32) if slot is None else slot
    if want_src and src is None:
        src = torch.empty(max(rows, 1), **i32)
    if want_invalid and num_invalid is None:
        num_invalid = torch.empty(1, **i32)
    need = layout_workspace_size(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(counts, "counts", torch.int32, E)
    _need(offsets, "offsets", torch.int32, E + 1)
    _need(slot, "slot", torch.int32, T * k)
    if src is not None:
        _need(src, "src", torch.int32, rows)
    if num_invalid is not None:
        _need(num_invalid, "num_invalid", torch.int32, 1)
    if num_dropped is not None:
        _need(num_dropped, "num_dropped", torch.int32, 1)
    _need(workspace, "workspace", torch.uint8)
    if alignment == 1 and capacity == 0 and num_dropped is None:
        st = lib().ep_layout(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(slot),
                             _ptr(src), _ptr(num_invalid), _ptr(workspace), workspace.numel(),
                             _stream(stream))
    else:
        st = lib().ep_layout_ex(_ptr(topk_idx), T, k, E, int(alignment), int(capacity),
                                _ptr(counts), _ptr(offsets), _ptr(slot), _ptr(src),
                                _ptr(num_invalid), _ptr(num_dropped), _ptr(workspace),
                                workspace.numel(), _stream(stream))
    _check(st, "ep_layout")
    return counts, offsets, slot, src, num_invalid


def ep_layout_noalloc(topk_idx: torch.Tensor, num_experts: int, counts: torch.Tensor,
                      offsets: torch.Tensor, slot: torch.Tensor, src: Optional[torch.Tensor] = None,
                      num_invalid: Optional[torch.Tensor] = None, stream=None):
    """ep_layout with the library's fixed per-device scratch: no workspace,
    and nothing allocated here or in the library (every output is the
    caller's).  Outputs as ep_layout; returns them."""
    _need(topk_idx, "topk_idx", torch.int64)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be 2-D [num_tokens, num_topk]")
    T, k = topk_idx.shape
    E = int(num_experts)
    _need(counts, "counts", torch.int32, E)
    _need(offsets, "offsets", torch.int32, E + 1)
    _need(slot, "slot", torch.int32, T * k)
    if src is not None:
        _need(src, "src", torch.int32, T * k)
    if num_invalid is not None:
        _need(num_invalid, "num_invalid", torch.int32, 1)
    st = lib().ep_layout_noalloc(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(slot),
                                 _ptr(src), _ptr(num_invalid), _stream(stream))
    _check(st, "ep_layout_noalloc")
    return counts, offsets, slot, src, num_invalid


# ---------------------------------------------------------------- dispatch --

def ep_dispatch(x: torch.Tensor, slot: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                *, fp8: bool = False, fmt: str = "e4m3", scale: str = "fp32", recv_x=None,
                recv_scales=None, recv_weights=None,
                want_weights: bool = False, rows: Optional[int] = None,
                trust_slots: bool = False, scale_ld: int = 0, stream=None):
    """Permute (bf16) or cast (fp8 e4m3 + per-128 fp32 scales) the rows of
    ``x`` (bf16 [T, H]) into the expert-grouped buffer named by ``slot``.

    With ``fp8`` the cast format is ``fmt`` ("e4m3" / "e5m2") and the scale
    ``scale`` ("fp32", "pow2", "ue8m0" -- the last gives uint8 scales);
    ``scale_ld`` > 0 stores the scales column-major, [H/128, scale_ld]
    (scale_ld >= rows, a multiple of 4 fp32 / 16 UE8M0 scales).

    Returns (recv_x, recv_scales or None, recv_weights or None); recv_x is
    bf16 [rows, H] or uint8 [rows, H].  ``rows`` is the layout's row bound
    (layout_max_rows; T*k for the compact layout) and output buffers given
    by the caller must hold that many, unless ``trust_slots`` says the
    caller knows every slot is below the rows it passed.
    """
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [num_tokens, hidden]")
    T, H = x.shape
    _need(slot, "slot", torch.int32)
    if slot.dim() != 2 or slot.shape[0] != T:
        raise ValueError("slot must be 2-D [num_tokens, num_topk]")
    k = slot.shape[1]
    R = T * k if rows is None else int(rows)
    dev = x.device
    if recv_x is None:
        recv_x = torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    sdt = torch.uint8 if scale == "ue8m0" else torch.float32
    nb = H // 128
    if scale_ld:
        if scale_ld < R:
            raise ValueError(f"scale_ld {scale_ld} is below the layout's {R} rows")
    if fp8 and recv_scales is None:
        recv_scales = torch.empty((nb, scale_ld) if scale_ld else (R, nb), dtype=sdt, device=dev)
    if want_weights and recv_weights is None:
        recv_weights = torch.empty(R, dtype=torch.float32, device=dev)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    cap = 0 if trust_slots else R
    _need(recv_x, "recv_x", torch.uint8 if fp8 else torch.bfloat16, cap * H)
    if recv_x.shape[-1] != H:
        raise ValueError("recv_x rows must have hidden elements")
    if recv_scales is not None:
        _need(recv_scales, "recv_scales", sdt, nb * scale_ld if scale_ld else cap * nb)
    if recv_weights is not None:
        _need(recv_weights, "recv_weights", torch.float32, cap)
    st = lib().ep_dispatch_ex(_ptr(x), T, H, k, _ptr(slot), _ptr(topk_weights),
                              _FORMATS[fmt] if fp8 else EP_OUT_BF16,
                              _SCALES[scale] if fp8 else EP_SCALE_FP32, _ptr(recv_x),
                              _ptr(recv_scales), _ptr(recv_weights), int(scale_ld),
                              _stream(stream))
    _check(st, "ep_dispatch")
    return recv_x, recv_scales, recv_weights


def ep_dispatch_colmajor_workspace_size(num_tokens: int, hidden: int, scale: str = "fp32") -> int:
    return int(lib().ep_dispatch_colmajor_workspace_size(int(num_tokens), int(hidden), _SCALES[scale]))


def ep_dispatch_colmajor_scales(x: torch.Tensor, slot: torch.Tensor, src: torch.Tensor,
                                topk_weights: Optional[torch.Tensor] = None, *, fmt: str = "e4m3",
                                scale: str = "fp32", scale_ld: int, rows: Optional[int] = None,
                                recv_x=None, recv_scales=None, recv_weights=None,
                                want_weights: bool = False, workspace=None, stream=None):
    """The 8-bit cast with column-major scales [H/128, scale_ld] written in
    two passes through a workspace (allocated here with torch when not
    given).  ``src`` is the layout's int32 source token of each of the
    ``rows`` receive rows (T*k by default).  Returns (recv_x uint8 [rows, H],
    recv_scales, recv_weights or None)."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [num_tokens, hidden]")
    T, H = x.shape
    _need(slot, "slot", torch.int32)
    if slot.dim() != 2 or slot.shape[0] != T:
        raise ValueError("slot must be 2-D [num_tokens, num_topk]")
    k = slot.shape[1]
    R = T * k if rows is None else int(rows)
    if scale_ld < R:
        raise ValueError(f"scale_ld {scale_ld} is below the {R} rows")
    _need(src, "src", torch.int32, R)
    dev = x.device
    sdt = torch.uint8 if scale == "ue8m0" else torch.float32
    nb = H // 128
    if recv_x is None:
        recv_x = torch.empty((R, H), dtype=torch.uint8, device=dev)
    if recv_scales is None:
        recv_scales = torch.empty((nb, scale_ld), dtype=sdt, device=dev)
    if want_weights and recv_weights is None:
        recv_weights = torch.empty(R, dtype=torch.float32, device=dev)
    need = ep_dispatch_colmajor_workspace_size(T, H, scale)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(recv_x, "recv_x", torch.uint8, R * H)
    _need(recv_scales, "recv_scales", sdt, nb * scale_ld)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    if recv_weights is not None:
        _need(recv_weights, "recv_weights", torch.float32, R)
    _need(workspace, "workspace", torch.uint8)
    st = lib().ep_dispatch_colmajor_scales(_ptr(x), T, H, k, _ptr(slot), _ptr(src),
                                           _ptr(topk_weights), _FORMATS[fmt], _SCALES[scale],
                                           _ptr(recv_x), _ptr(recv_scales), _ptr(recv_weights),
                                           int(scale_ld), R, _ptr(workspace), workspace.numel(),
                                           _stream(stream))
    _check(st, "ep_dispatch_colmajor_scales")
    return recv_x, recv_scales, recv_weights


def ep_dispatch_prequantized(x_q: torch.Tensor, x_scales: torch.Tensor, slot: torch.Tensor,
                             topk_weights: Optional[torch.Tensor] = None, *, recv_q=None,
                             recv_scales=None, recv_weights=None, want_weights: bool = False,
                             rows: Optional[int] = None, scale_ld: int = 0, stream=None):
    """Copy pre-quantized rows (uint8 [T, H]) and their fp32 scales
    ([T, H/128]) to the expert-grouped buffer (scales column-major
    [H/128, scale_ld] when scale_ld > 0).  Returns (recv_q, recv_scales,
    recv_weights or None)."""
    _need(x_q, "x_q", torch.uint8)
    _need(x_scales, "x_scales", torch.float32)
    _need(slot, "slot", torch.int32)
    if x_q.dim() != 2 or slot.dim() != 2 or slot.shape[0] != x_q.shape[0]:
        raise ValueError("x_q must be [T, H] and slot [T, k]")
    T, H = x_q.shape
    k = slot.shape[1]
    if x_scales.numel() < T * (H // 128):
        raise ValueError("x_scales must hold T * H/128 values")
    R = T * k if rows is None else int(rows)
    dev = x_q.device
    if recv_q is None:
        recv_q = torch.empty((R, H), dtype=torch.uint8, device=dev)
    nb = H // 128
    if scale_ld and scale_ld < R:
        raise ValueError(f"scale_ld {scale_ld} is below the layout's {R} rows")
    if recv_scales is None:
        recv_scales = torch.empty((nb, scale_ld) if scale_ld else (R, nb), dtype=torch.float32,
                                  device=dev)
    if want_weights and recv_weights is None:
        recv_weights = torch.empty(R, dtype=torch.float32, device=dev)
    _need(recv_q, "recv_q", torch.uint8, R * H)
    _need(recv_scales, "recv_scales", torch.float32, nb * scale_ld if scale_ld else R * nb)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    if recv_weights is not None:
        _need(recv_weights, "recv_weights", torch.float32, R)
    st = lib().ep_dispatch_prequantized(_ptr(x_q), _ptr(x_scales), T, H, k, _ptr(slot),
                                        _ptr(topk_weights), _ptr(recv_q), _ptr(recv_scales),
                                        _ptr(recv_weights), int(scale_ld), _stream(stream))
    _check(st, "ep_dispatch_prequantized")
    return recv_q, recv_scales, recv_weights


def ep_dispatch_prequantized_colmajor(x_q: torch.Tensor, x_scales: torch.Tensor,
                                      slot: torch.Tensor, src: torch.Tensor,
                                      topk_weights: Optional[torch.Tensor] = None, *,
                                      scale_ld: int, rows: Optional[int] = None, recv_q=None,
                                      recv_scales=None, recv_weights=None,
                                      want_weights: bool = False, stream=None):
    """The pre-quantized copy with column-major scales [H/128, scale_ld]
    written in two passes (the code rows, then the scale columns from
    x_scales).  ``src`` is the layout's int32 source token of each of the
    ``rows`` receive rows (T*k by default).  Returns (recv_q, recv_scales,
    recv_weights or None)."""
    _need(x_q, "x_q", torch.uint8)
    _need(x_scales, "x_scales", torch.float32)
    _need(slot, "slot", torch.int32)
    if x_q.dim() != 2 or slot.dim() != 2 or slot.shape[0] != x_q.shape[0]:
        raise ValueError("x_q must be [T, H] and slot [T, k]")
    T, H = x_q.shape
    k = slot.shape[1]
    nb = H // 128
    if x_scales.numel() < T * nb:
        raise ValueError("x_scales must hold T * H/128 values")
    R = T * k if rows is None else int(rows)
    if scale_ld < R:
        raise ValueError(f"scale_ld {scale_ld} is below the {R} rows")
    _need(src, "src", torch.int32, R)
    dev = x_q.device
    if recv_q is None:
        recv_q = torch.empty((R, H), dtype=torch.uint8, device=dev)
    if recv_scales is None:
        recv_scales = torch.empty((nb, scale_ld), dtype=torch.float32, device=dev)
    if want_weights and recv_weights is None:
        recv_weights = torch.empty(R, dtype=torch.float32, device=dev)
    _need(recv_q, "recv_q", torch.uint8, R * H)
    _need(recv_scales, "recv_scales", torch.float32, nb * scale_ld)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    if recv_weights is not None:
        _need(recv_weights, "recv_weights", torch.float32, R)
    st = lib().ep_dispatch_prequantized_colmajor(_ptr(x_q), _ptr(x_scales), T, H, k, _ptr(slot),
                                                 _ptr(src), _ptr(topk_weights), _ptr(recv_q),
                                                 _ptr(recv_scales), _ptr(recv_weights),
                                                 int(scale_ld), R, _stream(stream))
    _check(st, "ep_dispatch_prequantized_colmajor")
    return recv_q, recv_scales, recv_weights


# ----------------------------------------------------------------- combine --

def ep_combine(y: torch.Tensor, slot: torch.Tensor, topk_weights: Optional[torch.Tensor],
               *, out=None, rows: Optional[int] = None, trust_slots: bool = False,
               stream=None) -> torch.Tensor:
    """out[t] = bf16(sum_j w[t,j] * y[slot[t,j]]) for y bf16 [rows, H] and
    slot int32 [T, k]; ``topk_weights`` None means unit weights.  y must
    hold ``rows`` rows (the layout's bound, T*k by default) unless
    ``trust_slots`` says every slot is below its rows."""
    _need(y, "y", torch.bfloat16)
    _need(slot, "slot", torch.int32)
    if slot.dim() != 2 or y.dim() != 2:
        raise ValueError("slot must be [num_tokens, num_topk] and y [rows, hidden]")
    T, k = slot.shape
    H = y.shape[-1]
    R = T * k if rows is None else int(rows)
    if not trust_slots and y.shape[0] < R:
        raise ValueError(f"y has {y.shape[0]} rows, the layout may use {R}")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _need(out, "out", torch.bfloat16, T * H)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    st = lib().ep_combine(_ptr(y), _ptr(slot), _ptr(topk_weights), T, H, k, _ptr(out),
                          _stream(stream))
    _check(st, "ep_combine")
    return out


# ---------------------------------------------------------------- backward --

def ep_combine_backward(grad_out: torch.Tensor, y: Optional[torch.Tensor], slot: torch.Tensor,
                        topk_weights: Optional[torch.Tensor], *, grad_y=None,
                        grad_topk_weights=None, want_weight_grad: bool = True,
                        rows: Optional[int] = None, stream=None):
    """Gradients of ep_combine: returns (grad_y bf16 [rows, H],
    grad_topk_weights fp32 [T, k] or None).  The weight gradient needs y."""
    _need(grad_out, "grad_out", torch.bfloat16)
    _need(slot, "slot", torch.int32)
    if slot.dim() != 2 or grad_out.dim() != 2 or slot.shape[0] != grad_out.shape[0]:
        raise ValueError("grad_out must be [T, H] and slot [T, k]")
    T, H = grad_out.shape
    k = slot.shape[1]
    R = T * k if rows is None else int(rows)
    if grad_y is None:
        grad_y = torch.empty((R, H), dtype=torch.bfloat16, device=grad_out.device)
    _need(grad_y, "grad_y", torch.bfloat16, R * H)
    if y is not None:
        _need(y, "y", torch.bfloat16, R * H)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    if want_weight_grad and y is not None and grad_topk_weights is None:
        grad_topk_weights = torch.empty((T, k), dtype=torch.float32, device=grad_out.device)
    if grad_topk_weights is not None:
        _need(grad_topk_weights, "grad_topk_weights", torch.float32, T * k)
    st = lib().ep_combine_backward(_ptr(grad_out), _ptr(y), _ptr(slot), _ptr(topk_weights), T, H, k,
                                   _ptr(grad_y), _ptr(grad_topk_weights), _stream(stream))
    _check(st, "ep_combine_backward")
    return grad_y, grad_topk_weights


def ep_dispatch_backward(grad_recv: torch.Tensor, grad_recv_weights: Optional[torch.Tensor],
                         slot: torch.Tensor, *, grad_x=None, grad_topk_weights=None,
                         rows: Optional[int] = None, stream=None):
    """Gradients of ep_dispatch: returns (grad_x bf16 [T, H],
    grad_topk_weights fp32 [T, k] or None)."""
    _need(grad_recv, "grad_recv", torch.bfloat16)
    _need(slot, "slot", torch.int32)
    if slot.dim() != 2 or grad_recv.dim() != 2:
        raise ValueError("slot must be [T, k] and grad_recv [rows, H]")
    T, k = slot.shape
    H = grad_recv.shape[1]
    R = T * k if rows is None else int(rows)
    if grad_recv.shape[0] < R:
        raise ValueError(f"grad_recv has {grad_recv.shape[0]} rows, the layout may use {R}")
    if grad_x is None:
        grad_x = torch.empty((T, H), dtype=torch.bfloat16, device=grad_recv.device)
    _need(grad_x, "grad_x", torch.bfloat16, T * H)
    if grad_recv_weights is not None:
        _need(grad_recv_weights, "grad_recv_weights", torch.float32, R)
        if grad_topk_weights is None:
            grad_topk_weights = torch.empty((T, k), dtype=torch.float32, device=grad_recv.device)
        _need(grad_topk_weights, "grad_topk_weights", torch.float32, T * k)
    st = lib().ep_dispatch_backward(_ptr(grad_recv), _ptr(grad_recv_weights), _ptr(slot), T, H, k,
                                    _ptr(grad_x), _ptr(grad_topk_weights), _stream(stream))
    _check(st, "ep_dispatch_backward")
    return grad_x, grad_topk_weights


# ------------------------------------------------- per-(token, rank) path --

def ep_routing_map(topk_idx: torch.Tensor, num_experts: int, *, routing_map=None,
                   num_invalid=None, want_invalid: bool = True, stream=None):
    """Routing bitmap of ``topk_idx`` (int64 [T, k]): uint8 [T, ceil(E/8)],
    bit e % 8 of byte e // 8 set iff the token selects expert e.  Returns
    (routing_map, num_invalid int32 [1] or None)."""
    _need(topk_idx, "topk_idx", torch.int64)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be 2-D [num_tokens, num_topk]")
    T, k = topk_idx.shape
    E = int(num_experts)
    W = (E + 7) // 8
    dev = topk_idx.device
    if routing_map is None:
        routing_map = torch.empty((T, W), dtype=torch.uint8, device=dev)
    _need(routing_map, "routing_map", torch.uint8, T * W)
    if want_invalid and num_invalid is None:
        num_invalid = torch.empty(1, dtype=torch.int32, device=dev)
    if num_invalid is not None:
        _need(num_invalid, "num_invalid", torch.int32, 1)
    st = lib().ep_routing_map(_ptr(topk_idx), T, k, E, _ptr(routing_map), _ptr(num_invalid),
                              _stream(stream))
    _check(st, "ep_routing_map")
    return routing_map, num_invalid


def rank_layout_workspace_size(tokens_per_rank: int, num_experts: int, num_ranks: int) -> int:
    return int(lib().ep_rank_layout_workspace_size(int(tokens_per_rank), int(num_experts),
                                                   int(num_ranks)))


class RankLayout:
    """Outputs of :func:`ep_rank_layout` (device tensors)."""

    FIELDS = ("sparse_to_dense", "local_map", "recv_src", "recv_topk_idx", "expert_counts",
              "num_recv", "num_overflow")

    def __init__(self, **kw):
        self.__dict__.update(kw)


def ep_rank_layout(global_map: torch.Tensor, tokens_per_rank: int, num_experts: int,
                   num_ranks: int, rank: int, k_out: int, *, out: Optional[RankLayout] = None,
                   workspace=None, stream=None) -> RankLayout:
    """Metadata preprocessing of rank ``rank`` from the all-gathered routing
    map (uint8 [G*T, ceil(E/8)]).  Returns a RankLayout with
    sparse_to_dense int32 [T, G], local_map uint8 [G*T, E/G], recv_src int32
    [G*T], recv_topk_idx int64 [G*T, k_out], expert_counts int32 [E/G],
    num_recv int32 [1], num_overflow int32 [1]."""
    T, E, G = int(tokens_per_rank), int(num_experts), int(num_ranks)
    if G < 1 or E % G:
        raise ValueError("num_experts must be a multiple of num_ranks")
    El = E // G
    R = G * T
    W = (E + 7) // 8
    _need(global_map, "global_map", torch.uint8, R * W)
    dev = global_map.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = RankLayout(sparse_to_dense=torch.empty((T, G), **i32),
                         local_map=torch.empty((R, El), dtype=torch.uint8, device=dev),
                         recv_src=torch.empty(R, **i32),
                         recv_topk_idx=torch.empty((R, int(k_out)), dtype=torch.int64, device=dev),
                         expert_counts=torch.empty(El, **i32), num_recv=torch.empty(1, **i32),
                         num_overflow=torch.empty(1, **i32))
    _need(out.sparse_to_dense, "sparse_to_dense", torch.int32, T * G)
    _need(out.local_map, "local_map", torch.uint8, R * El)
    _need(out.recv_src, "recv_src", torch.int32, R)
    _need(out.recv_topk_idx, "recv_topk_idx", torch.int64, R * int(k_out))
    _need(out.expert_counts, "expert_counts", torch.int32, El)
    _need(out.num_recv, "num_recv", torch.int32, 1)
    if out.num_overflow is not None:
        _need(out.num_overflow, "num_overflow", torch.int32, 1)
    need = rank_layout_workspace_size(T, E, G)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    st = lib().ep_rank_layout(_ptr(global_map), T, E, G, int(rank), int(k_out),
                              _ptr(out.sparse_to_dense), _ptr(out.local_map), _ptr(out.recv_src),
                              _ptr(out.recv_topk_idx), _ptr(out.expert_counts), _ptr(out.num_recv),
                              _ptr(out.num_overflow), _ptr(workspace), workspace.numel(),
                              _stream(stream))
    _check(st, "ep_rank_layout")
    return out


def _ptr_table(tensors):
    arr = (ctypes.c_void_p * len(tensors))(*[None if t is None else t.data_ptr() for t in tensors])
    return arr, ctypes.addressof(arr)


def ep_dispatch_ranked(x: torch.Tensor, sparse_to_dense: torch.Tensor, dest_x, num_experts: int,
                       *, topk_idx: Optional[torch.Tensor] = None,
                       topk_weights: Optional[torch.Tensor] = None, dest_weights=None,
                       stream=None):
    """Send the rows of ``x`` (bf16 [T, H]) once to every rank that receives
    them: ``dest_x`` is a list of G bf16 [rows_d, H] tensors, ``dest_weights``
    None or a list of G fp32 [rows_d, k] tensors (entries may be None; needs
    ``topk_idx``).  Rows at or past the smallest rows_d are not written."""
    _need(x, "x", torch.bfloat16)
    _need(sparse_to_dense, "sparse_to_dense", torch.int32)
    if x.dim() != 2 or sparse_to_dense.dim() != 2 or sparse_to_dense.shape[0] != x.shape[0]:
        raise ValueError("x must be [T, H] and sparse_to_dense [T, G]")
    T, H = x.shape
    G = sparse_to_dense.shape[1]
    if len(dest_x) != G:
        raise ValueError("one destination buffer per rank")
    for d, t in enumerate(dest_x):
        _need(t, f"dest_x[{d}]", torch.bfloat16)
        if t.dim() != 2 or t.shape[1] != H:
            raise ValueError(f"dest_x[{d}] must be [rows, {H}]")
    rows = min(int(t.shape[0]) for t in dest_x)
    k = 1
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", torch.int64)
        if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
            raise ValueError("topk_idx must be [T, k]")
        k = topk_idx.shape[1]
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    wtab = None
    if dest_weights is not None:
        if topk_idx is None:
            raise ValueError("dest_weights needs topk_idx")
        if len(dest_weights) != G:
            raise ValueError("one weight buffer (or None) per rank")
        for d, t in enumerate(dest_weights):
            if t is not None:
                _need(t, f"dest_weights[{d}]", torch.float32, rows * k)
        wtab = _ptr_table(dest_weights)
    xtab = _ptr_table(dest_x)
    st = lib().ep_dispatch_ranked(_ptr(x), _ptr(topk_idx), _ptr(topk_weights), T, H, k,
                                  int(num_experts), G, _ptr(sparse_to_dense), xtab[1],
                                  None if wtab is None else wtab[1], rows, _stream(stream))
    _check(st, "ep_dispatch_ranked")
    return dest_x, dest_weights


def ep_dispatch_ranked_prequantized(x_q: torch.Tensor, x_scales: torch.Tensor,
                                    sparse_to_dense: torch.Tensor, dest_q, dest_scales,
                                    num_experts: int, *, topk_idx: Optional[torch.Tensor] = None,
                                    topk_weights: Optional[torch.Tensor] = None, dest_weights=None,
                                    stream=None):
    """Once-per-rank dispatch of 8-bit tokens: ``x_q`` uint8 [T, H] and
    ``x_scales`` fp32 [T, H/128] go to the G ranks' ``dest_q`` (uint8
    [rows_d, H]) and ``dest_scales`` (fp32 [rows_d, H/128]); weights as
    ep_dispatch_ranked.  Rows at or past the smallest rows_d are not
    written."""
    _need(x_q, "x_q", torch.uint8)
    _need(x_scales, "x_scales", torch.float32)
    _need(sparse_to_dense, "sparse_to_dense", torch.int32)
    if x_q.dim() != 2 or sparse_to_dense.dim() != 2 or sparse_to_dense.shape[0] != x_q.shape[0]:
        raise ValueError("x_q must be [T, H] and sparse_to_dense [T, G]")
    T, H = x_q.shape
    nb = H // 128
    _need(x_scales, "x_scales", torch.float32, T * nb)
    G = sparse_to_dense.shape[1]
    if len(dest_q) != G or len(dest_scales) != G:
        raise ValueError("one code and one scale buffer per rank")
    for d in range(G):
        _need(dest_q[d], f"dest_q[{d}]", torch.uint8)
        if dest_q[d].dim() != 2 or dest_q[d].shape[1] != H:
            raise ValueError(f"dest_q[{d}] must be [rows, {H}]")
        _need(dest_scales[d], f"dest_scales[{d}]", torch.float32)
    rows = min(int(t.shape[0]) for t in dest_q)
    for d in range(G):
        _need(dest_scales[d], f"dest_scales[{d}]", torch.float32, rows * nb)
    k = 1
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", torch.int64)
        k = topk_idx.shape[1]
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    wtab = None
    if dest_weights is not None:
        if topk_idx is None or len(dest_weights) != G:
            raise ValueError("dest_weights needs topk_idx and one buffer (or None) per rank")
        for d, t in enumerate(dest_weights):
            if t is not None:
                _need(t, f"dest_weights[{d}]", torch.float32, rows * k)
        wtab = _ptr_table(dest_weights)
    qtab = _ptr_table(dest_q)
    stab = _ptr_table(dest_scales)
    st = lib().ep_dispatch_ranked_prequantized(_ptr(x_q), _ptr(x_scales), _ptr(topk_idx),
                                               _ptr(topk_weights), T, H, k, int(num_experts), G,
                                               _ptr(sparse_to_dense), qtab[1], stab[1],
                                               None if wtab is None else wtab[1], rows,
                                               _stream(stream))
    _check(st, "ep_dispatch_ranked_prequantized")
    return dest_q, dest_scales, dest_weights


def ep_dispatch_ranked_fp8(x: torch.Tensor, sparse_to_dense: torch.Tensor, dest_q, dest_scales,
                           num_experts: int, *, fmt: str = "e4m3", scale: str = "fp32",
                           topk_idx: Optional[torch.Tensor] = None,
                           topk_weights: Optional[torch.Tensor] = None, dest_weights=None,
                           stream=None):
    """Once-per-rank dispatch with the 8-bit cast on the way: ``x`` bf16
    [T, H] (H a multiple of 128) is cast as ep_dispatch casts it (``fmt``
    "e4m3" / "e5m2", ``scale`` "fp32" / "pow2" / "ue8m0") and each token's
    codes and scales go to the G ranks' ``dest_q`` (uint8 [rows_d, H]) and
    ``dest_scales`` ([rows_d, H/128], fp32, or uint8 for "ue8m0"); weights as
    ep_dispatch_ranked.  Rows at or past the smallest rows_d are not
    written."""
    _need(x, "x", torch.bfloat16)
    _need(sparse_to_dense, "sparse_to_dense", torch.int32)
    if x.dim() != 2 or sparse_to_dense.dim() != 2 or sparse_to_dense.shape[0] != x.shape[0]:
        raise ValueError("x must be [T, H] and sparse_to_dense [T, G]")
    T, H = x.shape
    nb = H // 128
    G = sparse_to_dense.shape[1]
    sdt = torch.uint8 if scale == "ue8m0" else torch.float32
    if len(dest_q) != G or len(dest_scales) != G:
        raise ValueError("one code and one scale buffer per rank")
    for d in range(G):
        _need(dest_q[d], f"dest_q[{d}]", torch.uint8)
        if dest_q[d].dim() != 2 or dest_q[d].shape[1] != H:
            raise ValueError(f"dest_q[{d}] must be [rows, {H}]")
    rows = min(int(t.shape[0]) for t in dest_q)
    for d in range(G):
        _need(dest_scales[d], f"dest_scales[{d}]", sdt, rows * nb)
    k = 1
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", torch.int64)
        k = topk_idx.shape[1]
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, T * k)
    wtab = None
    if dest_weights is not None:
        if topk_idx is None or len(dest_weights) != G:
            raise ValueError("dest_weights needs topk_idx and one buffer (or None) per rank")
        for d, t in enumerate(dest_weights):
            if t is not None:
                _need(t, f"dest_weights[{d}]", torch.float32, rows * k)
        wtab = _ptr_table(dest_weights)
    qtab = _ptr_table(dest_q)
    stab = _ptr_table(dest_scales)
    st = lib().ep_dispatch_ranked_fp8(_ptr(x), _ptr(topk_idx), _ptr(topk_weights), T, H, k,
                                      int(num_experts), G, _ptr(sparse_to_dense), _FORMATS[fmt],
                                      _SCALES[scale], qtab[1], stab[1],
                                      None if wtab is None else wtab[1], rows, _stream(stream))
    _check(st, "ep_dispatch_ranked_fp8")


def _fused_permute_tables(G, T, k, R, src_topk_idx, src_topk_weights, recv_weights):
    itab = wtab = None
    if recv_weights is not None:
        _need(recv_weights, "recv_weights", torch.float32, R)
        if src_topk_idx is None or len(src_topk_idx) != G:
            raise ValueError("recv_weights needs src_topk_idx for every rank")
        for d, t in enumerate(src_topk_idx):
            _need(t, f"src_topk_idx[{d}]", torch.int64, T * k)
        itab = _ptr_table(src_topk_idx)
        if src_topk_weights is not None:
            for d, t in enumerate(src_topk_weights):
                if t is not None:
                    _need(t, f"src_topk_weights[{d}]", torch.float32, T * k)
            wtab = _ptr_table(src_topk_weights)
    return itab, wtab


def _fused_permute_routing(G, T, recv_src, recv_topk_idx, slot, num_recv):
    _need(recv_src, "recv_src", torch.int32, G * T)
    _need(recv_topk_idx, "recv_topk_idx", torch.int64)
    _need(slot, "slot", torch.int32)
    if slot.dim() != 2 or slot.shape[0] != G * T or recv_topk_idx.shape != slot.shape:
        raise ValueError("slot and recv_topk_idx must be [G*T, k]")
    if num_recv is not None:
        _need(num_recv, "num_recv", torch.int32, 1)
    return slot.shape[1]


def ep_dispatch_fused_permute(src_x, recv_src: torch.Tensor, recv_topk_idx: torch.Tensor,
                              slot: torch.Tensor, num_experts: int, rank: int, *, rows: int,
                              src_topk_idx=None, src_topk_weights=None, num_recv=None,
                              recv_x=None, recv_weights=None, want_weights: bool = False,
                              stream=None):
    """The receiving rank's dispatch with the permute fused in: ``src_x`` is
    a list of the G ranks' tokens (bf16 [T, H]); ``recv_src`` /
    ``recv_topk_idx`` come from ep_rank_layout and ``slot`` from ep_layout of
    recv_topk_idx over E/G experts; ``rows`` is the expert-grouped buffer's
    row count.  Weights need ``src_topk_idx`` (list of int64 [T, k]) and
    optionally ``src_topk_weights`` (list of fp32 [T, k] or None).
    ``num_recv`` (int32 [1] on the device, from ep_rank_layout) bounds the
    rows visited; None visits all G*T.  Returns (recv_x bf16 [rows, H],
    recv_weights fp32 [rows] or None)."""
    G = len(src_x)
    for d, t in enumerate(src_x):
        _need(t, f"src_x[{d}]", torch.bfloat16)
    T, H = src_x[0].shape
    for t in src_x:
        if tuple(t.shape) != (T, H):
            raise ValueError("every src_x must be [T, H]")
    k = _fused_permute_routing(G, T, recv_src, recv_topk_idx, slot, num_recv)
    R = int(rows)
    dev = src_x[0].device
    if recv_x is None:
        recv_x = torch.empty((max(R, 1), H), dtype=torch.bfloat16, device=dev)
    _need(recv_x, "recv_x", torch.bfloat16, R * H)
    if want_weights and recv_weights is None:
        recv_weights = torch.empty(max(R, 1), dtype=torch.float32, device=dev)
    itab, wtab = _fused_permute_tables(G, T, k, R, src_topk_idx, src_topk_weights, recv_weights)
    xtab = _ptr_table(src_x)
    st = lib().ep_dispatch_fused_permute(xtab[1], None if itab is None else itab[1],
                                         None if wtab is None else wtab[1], T, H, k,
                                         int(num_experts), G, int(rank), _ptr(recv_src),
                                         _ptr(recv_topk_idx), _ptr(num_recv), _ptr(slot), R,
                                         _ptr(recv_x),
                                         _ptr(recv_weights), _stream(stream))
    _check(st, "ep_dispatch_fused_permute")
    return recv_x, recv_weights


def ep_dispatch_fused_permute_prequantized(src_q, src_scales, recv_src: torch.Tensor,
                                           recv_topk_idx: torch.Tensor, slot: torch.Tensor,
                                           num_experts: int, rank: int, *, rows: int,
                                           src_topk_idx=None, src_topk_weights=None,
                                           num_recv=None, recv_q=None, recv_scales=None,
                                           recv_weights=None, want_weights: bool = False,
                                           stream=None):
    """ep_dispatch_fused_permute for tokens the senders already cast to
    8 bits: ``src_q`` is a list of the G ranks' code rows (uint8 [T, H], H a
    multiple of 128) and ``src_scales`` their scale rows (fp32 [T, H/128]).
    Returns (recv_q uint8 [rows, H], recv_scales fp32 [rows, H/128],
    recv_weights fp32 [rows] or None)."""
    G = len(src_q)
    if len(src_scales) != G:
        raise ValueError("one scale tensor per rank")
    for d, t in enumerate(src_q):
        _need(t, f"src_q[{d}]", torch.uint8)
    T, H = src_q[0].shape
    nb = H // 128
    for d in range(G):
        if tuple(src_q[d].shape) != (T, H):
            raise ValueError("every src_q must be [T, H]")
        _need(src_scales[d], f"src_scales[{d}]", torch.float32, T * nb)
    k = _fused_permute_routing(G, T, recv_src, recv_topk_idx, slot, num_recv)
    R = int(rows)
    dev = src_q[0].device
    if recv_q is None:
        recv_q = torch.empty((max(R, 1), H), dtype=torch.uint8, device=dev)
    if recv_scales is None:
        recv_scales = torch.empty((max(R, 1), max(nb, 1)), dtype=torch.float32, device=dev)
    _need(recv_q, "recv_q", torch.uint8, R * H)
    _need(recv_scales, "recv_scales", torch.float32, R * nb)
    if want_weights and recv_weights is None:
        recv_weights = torch.empty(max(R, 1), dtype=torch.float32, device=dev)
    itab, wtab = _fused_permute_tables(G, T, k, R, src_topk_idx, src_topk_weights, recv_weights)
    qtab = _ptr_table(src_q)
    stab = _ptr_table(src_scales)
    st = lib().ep_dispatch_fused_permute_prequantized(
        qtab[1], stab[1], None if itab is None else itab[1], None if wtab is None else wtab[1], T,
        H, k, int(num_experts), G, int(rank), _ptr(recv_src), _ptr(recv_topk_idx),
        _ptr(num_recv), _ptr(slot), R, _ptr(recv_q), _ptr(recv_scales), _ptr(recv_weights),
        _stream(stream))
    _check(st, "ep_dispatch_fused_permute_prequantized")
    return recv_q, recv_scales, recv_weights


def ep_combine_ranked(src_y, sparse_to_dense: torch.Tensor, *, out=None, stream=None) -> torch.Tensor:
    """out[t] = bf16(sum over ranks d holding token t of src_y[d][row]) with
    ``src_y`` a list of G bf16 [rows_d, H] tensors; rows at or past the
    smallest rows_d read as 0."""
    _need(sparse_to_dense, "sparse_to_dense", torch.int32)
    if sparse_to_dense.dim() != 2:
        raise ValueError("sparse_to_dense must be [T, G]")
    T, G = sparse_to_dense.shape
    if len(src_y) != G:
        raise ValueError("one source buffer per rank")
    H = None
    for d, t in enumerate(src_y):
        _need(t, f"src_y[{d}]", torch.bfloat16)
        if t.dim() != 2 or (H is not None and t.shape[1] != H):
            raise ValueError("every src_y must be [rows, H] with the same H")
        H = t.shape[1]
    rows = min(int(t.shape[0]) for t in src_y)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=sparse_to_dense.device)
    _need(out, "out", torch.bfloat16, T * H)
    ytab = _ptr_table(src_y)
    st = lib().ep_combine_ranked(ytab[1], rows, _ptr(sparse_to_dense), T, H, G, _ptr(out),
                                 _stream(stream))
    _check(st, "ep_combine_ranked")
    return out


def ep_dispatch_ranked_backward(sparse_to_dense: torch.Tensor, num_experts: int, *,
                                grad_recv_x=None, grad_recv_weights=None,
                                topk_idx: Optional[torch.Tensor] = None, grad_x=None,
                                grad_topk_weights=None, stream=None):
    """Backward of ep_dispatch_ranked for this rank's tokens.
    ``grad_recv_x``: None or a list of G bf16 [rows, H] row gradients (gives
    grad_x [T, H], the combine over ranks); ``grad_recv_weights``: None or a
    list of G fp32 [rows, k] weight gradients (entries may be None; gives
    grad_topk_weights [T, k], needs ``topk_idx``).  Rows at or past the
    smallest buffer's rows read as 0.  Returns (grad_x, grad_topk_weights)."""
    _need(sparse_to_dense, "sparse_to_dense", torch.int32)
    if sparse_to_dense.dim() != 2:
        raise ValueError("sparse_to_dense must be [T, G]")
    T, G = sparse_to_dense.shape
    dev = sparse_to_dense.device
    rows = None
    H = 0
    k = 1
    xtab = wtab = None
    if grad_recv_x is not None:
        if len(grad_recv_x) != G:
            raise ValueError("one row-gradient buffer per rank")
        for d, t in enumerate(grad_recv_x):
            _need(t, f"grad_recv_x[{d}]", torch.bfloat16)
            if t.dim() != 2 or (H and t.shape[1] != H):
                raise ValueError("every grad_recv_x must be [rows, H] with the same H")
            H = t.shape[1]
        rows = min(int(t.shape[0]) for t in grad_recv_x)
        if grad_x is None:
            grad_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        _need(grad_x, "grad_x", torch.bfloat16, T * H)
        xtab = _ptr_table(grad_recv_x)
    if grad_recv_weights is not None:
        if topk_idx is None:
            raise ValueError("grad_recv_weights needs topk_idx")
        _need(topk_idx, "topk_idx", torch.int64, T)
        k = topk_idx.shape[1]
        if len(grad_recv_weights) != G:
            raise ValueError("one weight-gradient buffer per rank")
        wrows = []
        for d, t in enumerate(grad_recv_weights):
            if t is None:
                continue
            _need(t, f"grad_recv_weights[{d}]", torch.float32)
            if t.dim() != 2 or t.shape[1] != k:
                raise ValueError("every grad_recv_weights must be [rows, k]")
            wrows.append(int(t.shape[0]))
        if wrows:
            rows = min(wrows + ([rows] if rows is not None else []))
        if grad_topk_weights is None:
            grad_topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
        _need(grad_topk_weights, "grad_topk_weights", torch.float32, T * k)
        wtab = _ptr_table(grad_recv_weights)
    st = lib().ep_dispatch_ranked_backward(
        None if xtab is None else xtab[1], None if wtab is None else wtab[1], rows or 0,
        _ptr(topk_idx), _ptr(sparse_to_dense), T, H or 8, k, int(num_experts), G,
        _ptr(grad_x) if xtab is not None else None,
        _ptr(grad_topk_weights) if wtab is not None else None, _stream(stream))
    _check(st, "ep_dispatch_ranked_backward")
    return (grad_x if xtab is not None else None,
            grad_topk_weights if wtab is not None else None)


# ------------------------------------------------------ C-ABI names, 1:1 --
# Every function include/ep.h declares is reachable here under its own name.
# The helpers above keep short names and ep_layout / ep_dispatch take the
# _ex arguments as keywords; these are the same calls under the header's
# names.

ep_version = version
ep_status_string = status_string
ep_last_error = last_error
ep_layout_workspace_size = layout_workspace_size
ep_layout_max_rows = layout_max_rows
ep_rank_layout_workspace_size = rank_layout_workspace_size


def ep_layout_ex(topk_idx: torch.Tensor, num_experts: int, alignment: int, capacity: int, **kw):
    """ep_layout with segment starts aligned to ``alignment`` rows, or a fixed
    ``capacity`` rows per expert (overflow dropped, counted in num_dropped)."""
    return ep_layout(topk_idx, num_experts, alignment=alignment, capacity=capacity, **kw)


def ep_dispatch_ex(x: torch.Tensor, slot: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                   *, out_dtype: str = "e4m3", scale: str = "fp32", scale_ld: int = 0, **kw):
    """ep_dispatch with the output type named: ``out_dtype`` "bf16" (a copy),
    "e4m3" or "e5m2" (a cast with ``scale`` "fp32", "pow2" or "ue8m0" block
    scales, row-major or, with ``scale_ld`` > 0, column-major)."""
    if out_dtype == "bf16":
        if scale_ld:
            raise ValueError("bf16 output takes no scale_ld")
        return ep_dispatch(x, slot, topk_weights, **kw)
    if out_dtype not in _FORMATS:
        raise ValueError(f"unknown out_dtype {out_dtype!r}")
    return ep_dispatch(x, slot, topk_weights, fp8=True, fmt=out_dtype, scale=scale,
                       scale_ld=scale_ld, **kw)
