"""C ABI checks that need no GPU: the library loads, exports every symbol
include/ep.h declares, and rejects bad arguments on the host before
launching anything (these calls fail validation, so no HIP call is made)."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from combine_ep_layout_04_amd import ep
from combine_ep_layout_04_amd.build import ROOT

HEADER = os.path.join(ROOT, "include", "ep.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(ep.SYMBOLS)


@pytest.mark.parametrize("compiler,flags", [
    ("gcc", ["-x", "c", "-std=c99", "-pedantic-errors"]),
    ("g++", ["-x", "c++", "-std=c++17", "-pedantic-errors"]),
])
def test_header_is_plain_c(tmp_path, compiler, flags):
    # the header compiles as strict C99 and as C++ on its own (no HIP or
    # torch headers), and every declared function can be named from C
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    names = declared_functions()
    src = tmp_path / "use_ep.c"
    src.write_text('#include "ep.h"\n'
                   "typedef void (*fn)(void);\n"
                   "fn table[] = {\n" + "".join(f"    (fn){n},\n" for n in names) + "};\n")
    r = subprocess.run([compiler, *flags, "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-I", os.path.dirname(HEADER), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_binding_has_every_declared_name():
    # the Python binding offers each entry point under the header's name
    for name in declared_functions():
        assert callable(getattr(ep, name, None)), name
    assert ep.ep_layout_workspace_size(4096, 8, 64) == ep.layout_workspace_size(4096, 8, 64)
    assert ep.ep_layout_max_rows(100, 4, 8, 16, 0) == ep.layout_max_rows(100, 4, 8, 16, 0)
    assert ep.ep_status_string(1) == "EP_INVALID_ARGUMENT"


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(ep.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert ep.version() >> 16 == 1
    assert ep.status_string(0) == "EP_SUCCESS"
    assert ep.status_string(1) == "EP_INVALID_ARGUMENT"
    assert ep.status_string(2) == "EP_UNSUPPORTED"
    assert ep.status_string(3) == "EP_RUNTIME_ERROR"
    assert ep.status_string(99) == "EP_UNKNOWN_STATUS"


def test_workspace_size():
    # one int32 per (chunk, expert) plus one per chunk, chunks padded to a
    # multiple of 4, 256-byte aligned; up to 65536 pairs about 64 chunks of
    # at least 256 pairs, beyond that chunks of 1024 pairs until there would
    # be more than 256 of them
    def want(chunks, E):
        cp = (chunks + 3) // 4 * 4
        return ((cp * E + cp) * 4 + 255) // 256 * 256
    assert ep.layout_workspace_size(8192, 8, 256) == want(64, 256) == 64 * 257 * 4
    assert ep.layout_workspace_size(0, 8, 256) == want(1, 256)
    assert ep.layout_workspace_size(1000, 3, 7) == want(12, 7)          # 256-pair chunks
    assert ep.layout_workspace_size(4096, 4, 64) == want(64, 64)        # 256-pair chunks
    assert ep.layout_workspace_size(4096, 8, 64) == want(64, 64)        # 512-pair chunks
    assert ep.layout_workspace_size(65536, 8, 256) == want(256, 256)     # 2048-pair chunks
    assert ep.layout_workspace_size(65537, 8, 256) == want(228, 256)     # 2304-pair chunks
    assert ep.layout_workspace_size(10, 0, 8) == 0
    assert ep.layout_workspace_size(10, 2, 0) == 0
    assert ep.layout_workspace_size(10, 2, 1025) == 0
    assert ep.layout_workspace_size(1 << 28, 8, 8) == 0  # pairs >= 2^31


FAKE = 0x100000  # 16- and 256-byte aligned, never dereferenced by these calls

# The calls below hand the library fake device pointers and expect a host-side
# rejection.  Should a case ever pass validation by mistake it would launch a
# kernel on them, so they run only where no GPU is visible.
no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0,
    reason="fake pointers must never reach a launch on a real GPU")


@no_gpu
@pytest.mark.parametrize("args,code", [
    # (topk_idx, T, k, E, counts, offsets, slot, src, invalid, ws, ws_bytes)
    ((FAKE, 4, 2, 0, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20), 1),       # E < 1
    ((FAKE, 4, 2, 1025, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20), 1),    # E too large
    ((FAKE, 4, 0, 8, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20), 1),       # k < 1
    ((FAKE, 4, 65, 8, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20), 1),      # k too large
    ((FAKE, -1, 2, 8, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20), 1),      # T < 0
    ((FAKE, 1 << 28, 8, 8, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40), 2),  # pairs >= 2^31
    ((None, 4, 2, 8, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20), 1),       # no topk_idx
    ((FAKE, 4, 2, 8, None, FAKE, FAKE, None, None, FAKE, 1 << 20), 1),       # no counts
    ((FAKE, 4, 2, 8, FAKE, FAKE, None, None, None, FAKE, 1 << 20), 1),       # no slot
    ((FAKE, 4, 2, 8, FAKE, FAKE, FAKE, None, None, None, 1 << 20), 1),       # no workspace
    ((FAKE, 4, 2, 8, FAKE, FAKE, FAKE, None, None, FAKE + 16, 1 << 20), 1),  # ws misaligned
    ((FAKE, 4, 2, 8, FAKE, FAKE, FAKE, None, None, FAKE, 16), 1),            # ws too small
    ((FAKE + 4, 4, 2, 8, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20), 1),   # idx misaligned
])
def test_layout_rejects(args, code):
    st = ep.lib().ep_layout(*args, None)
    assert st == code, ep.last_error()
    assert ep.last_error()


@no_gpu
@pytest.mark.parametrize("args,code", [
    # (topk_idx, T, k, E, counts, offsets, slot, src, invalid): invalid shapes
    # are rejected before the library looks up its scratch
    ((FAKE, 4, 2, 0, FAKE, FAKE, FAKE, None, None), 1),          # E < 1
    ((FAKE, 4, 2, 1025, FAKE, FAKE, FAKE, None, None), 1),       # E too large
    ((FAKE, 4, 0, 8, FAKE, FAKE, FAKE, None, None), 1),          # k < 1
    ((FAKE, -1, 2, 8, FAKE, FAKE, FAKE, None, None), 1),         # T < 0
    ((FAKE, 1 << 28, 8, 8, FAKE, FAKE, FAKE, None, None), 2),    # pairs >= 2^31
])
def test_layout_noalloc_rejects(args, code):
    st = ep.lib().ep_layout_noalloc(*args, None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def test_layout_noalloc_scratch_covers_every_accepted_shape():
    # the fixed scratch equals the largest workspace ep_layout can ask for:
    # 256 chunks (the most the layout cuts) of EP_MAX_EXPERTS counts
    L = ep.lib()
    biggest = max(L.ep_layout_workspace_size(T, k, ep.EP_MAX_EXPERTS)
                  for T, k in ((1 << 20, 8), ((1 << 31) // 64 - 1, 64), (1 << 26, 16)))
    assert biggest == (256 * 1024 + 256) * 4
    header = open(HEADER).read()
    assert "#define EP_LAYOUT_NOALLOC_SCRATCH_BYTES ((size_t)(256 * 1024 + 256) * 4)" in header


@no_gpu
@pytest.mark.parametrize("args,code", [
    # (x, T, H, k, slot, w, out_dtype, recv_x, recv_scales, recv_w)
    ((FAKE, 4, 7, 2, FAKE, None, 0, FAKE, None, None), 1),          # H % 8
    ((FAKE, 4, 0, 2, FAKE, None, 0, FAKE, None, None), 1),          # H < 1
    ((FAKE, 4, 65544, 2, FAKE, None, 0, FAKE, None, None), 1),      # H too large
    ((FAKE, 4, 136, 2, FAKE, None, 1, FAKE, FAKE, None), 1),        # fp8 needs H % 128
    ((FAKE, 4, 256, 2, FAKE, None, 1, FAKE, None, None), 1),        # fp8 needs scales
    ((FAKE, 4, 256, 2, FAKE, None, 0, FAKE, FAKE, None), 1),        # bf16 with scales
    ((FAKE, 4, 256, 2, FAKE, None, 2, FAKE, None, None), 1),        # unknown dtype
    ((FAKE, 4, 256, 0, FAKE, None, 0, FAKE, None, None), 1),        # k < 1
    ((None, 4, 256, 2, FAKE, None, 0, FAKE, None, None), 1),        # no x
    ((FAKE, 4, 256, 2, None, None, 0, FAKE, None, None), 1),        # no slot
    ((FAKE, 4, 256, 2, FAKE, None, 0, None, None, None), 1),        # no recv_x
    ((FAKE + 8, 4, 256, 2, FAKE, None, 0, FAKE, None, None), 1),    # x misaligned
    ((FAKE, 4, 256, 2, FAKE, None, 0, FAKE + 2, None, None), 1),    # recv misaligned
    ((FAKE, 4, 256, 2, FAKE, None, 0, FAKE, None, FAKE), 1),        # recv_w without w
    ((FAKE, 1 << 28, 256, 8, FAKE, None, 0, FAKE, None, None), 2),  # pairs >= 2^31
])
def test_dispatch_rejects(args, code):
    st = ep.lib().ep_dispatch(*args, None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def test_dispatch_and_combine_zero_tokens_are_noops():
    assert ep.lib().ep_dispatch(None, 0, 256, 2, None, None, 0, None, None, None, None) == 0
    assert ep.lib().ep_combine(None, None, None, 0, 256, 2, None, None) == 0
    assert ep.last_error() == ""


@no_gpu
@pytest.mark.parametrize("args,code", [
    # (y, slot, w, T, H, k, out)
    ((FAKE, FAKE, None, 4, 12, 2, FAKE), 1),        # H % 8
    ((FAKE, FAKE, None, 4, 256, 65, FAKE), 1),      # k too large
    ((FAKE, FAKE, None, -3, 256, 2, FAKE), 1),      # T < 0
    ((None, FAKE, None, 4, 256, 2, FAKE), 1),       # no y
    ((FAKE, None, None, 4, 256, 2, FAKE), 1),       # no slot
    ((FAKE, FAKE, None, 4, 256, 2, None), 1),       # no out
    ((FAKE + 4, FAKE, None, 4, 256, 2, FAKE), 1),   # y misaligned
    ((FAKE, FAKE, None, 4, 256, 2, FAKE + 8), 1),   # out misaligned
])
def test_combine_rejects(args, code):
    st = ep.lib().ep_combine(*args, None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ep, "_lib", None)
    monkeypatch.setattr(ep, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ep.lib()


def test_layout_max_rows():
    assert ep.layout_max_rows(8192, 8, 256) == 65536
    assert ep.layout_max_rows(8192, 8, 256, 128) == 65536 + 256 * 127
    assert ep.layout_max_rows(3, 1, 256, 128) == 3 + 3 * 127       # only 3 experts can be hit
    assert ep.layout_max_rows(8192, 8, 256, 1, 512) == 256 * 512
    assert ep.layout_max_rows(8192, 8, 256, 128, 512) == 256 * 512
    assert ep.layout_max_rows(8192, 8, 256, 128, 500) == -1          # capacity % alignment
    assert ep.layout_max_rows(8192, 8, 256, 0) == -1
    assert ep.layout_max_rows(8192, 8, 256, 4097) == -1
    assert ep.layout_max_rows(8192, 8, 256, 1, -1) == -1


@no_gpu
@pytest.mark.parametrize("A,cap,T,code", [
    (0, 0, 4, 1),                 # alignment < 1
    (4097, 0, 4, 1),              # alignment too large
    (4, 6, 4, 1),                 # capacity not a multiple of alignment
    (1, -2, 4, 1),                # negative capacity
    (4096, 0, (1 << 30) - 1, 2),  # 2^31-2 pairs + 256*4095 padding rows >= 2^31
    (1, 1 << 24, 4, 2),           # E * capacity >= 2^31
])
def test_layout_ex_rejects(A, cap, T, code):
    st = ep.lib().ep_layout_ex(FAKE, T, 2, 256, A, cap, FAKE, FAKE, FAKE, None, None, None,
                               FAKE, 1 << 30, None)
    assert st == code, ep.last_error()


# ---- per-(token, rank) path

def test_rank_layout_workspace_size():
    # per chunk: one int32 per rank, one per local expert and one overflow
    # count, 256-byte aligned; chunks hold 256 global tokens until there
    # would be more than 256 of them
    def want(chunks, G, El):
        return (chunks * (G + El + 1) * 4 + 255) // 256 * 256
    assert ep.rank_layout_workspace_size(8192, 256, 8) == want(256, 8, 32)
    assert ep.rank_layout_workspace_size(0, 256, 8) == want(1, 8, 32)
    assert ep.rank_layout_workspace_size(8192, 256, 1) == want(32, 1, 256)
    assert ep.rank_layout_workspace_size(65536, 64, 64) == want(256, 64, 1)   # 16384-token chunks
    assert ep.rank_layout_workspace_size(65537, 64, 64) == want(253, 64, 1)   # 16640-token chunks
    assert ep.rank_layout_workspace_size(10, 256, 3) == 0        # E % G
    assert ep.rank_layout_workspace_size(10, 256, 65) == 0
    assert ep.rank_layout_workspace_size(10, 0, 1) == 0
    assert ep.rank_layout_workspace_size(-1, 8, 2) == 0


@no_gpu
@pytest.mark.parametrize("args,code", [
    # (topk_idx, T, k, E, routing_map, num_invalid)
    ((FAKE, 4, 2, 0, FAKE, None), 1),             # E < 1
    ((FAKE, 4, 2, 1025, FAKE, None), 1),          # E too large
    ((FAKE, 4, 0, 8, FAKE, None), 1),             # k < 1
    ((FAKE, -1, 2, 8, FAKE, None), 1),            # T < 0
    ((FAKE, 1 << 28, 8, 8, FAKE, None), 2),       # pairs >= 2^31
    ((None, 4, 2, 8, FAKE, None), 1),             # no topk_idx
    ((FAKE, 4, 2, 8, None, None), 1),             # no map
    ((FAKE + 4, 4, 2, 8, FAKE, None), 1),         # idx misaligned
    ((FAKE, 4, 2, 8, FAKE, FAKE + 2), 1),         # num_invalid misaligned
])
def test_routing_map_rejects(args, code):
    st = ep.lib().ep_routing_map(*args, None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def _rank_layout_args(**over):
    a = dict(map=FAKE, T=4, E=8, G=2, rank=0, k_out=2, s2d=FAKE, lm=FAKE, src=FAKE, rti=FAKE,
             counts=FAKE, nrecv=FAKE, novf=None, ws=FAKE, ws_bytes=1 << 20)
    a.update(over)
    return tuple(a.values())


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(G=0), 1), (dict(G=65, E=130), 1), (dict(E=9), 1), (dict(E=1026, G=2), 1),
    (dict(rank=-1), 1), (dict(rank=2), 1), (dict(k_out=0), 1), (dict(k_out=65), 1),
    (dict(T=-1), 1), (dict(T=1 << 28, G=8), 2),
    (dict(counts=None), 1), (dict(nrecv=None), 1), (dict(map=None), 1), (dict(s2d=None), 1),
    (dict(lm=None), 1), (dict(src=None), 1), (dict(rti=None), 1),
    (dict(lm=FAKE + 1), 1), (dict(s2d=FAKE + 2), 1), (dict(rti=FAKE + 4), 1),
    (dict(ws=None), 1), (dict(ws=FAKE + 16), 1), (dict(ws_bytes=16), 1),
])
def test_rank_layout_rejects(over, code):
    st = ep.lib().ep_rank_layout(*_rank_layout_args(**over), None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def _table(*ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return arr


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(H=12), 1), (dict(k=0), 1), (dict(G=65, E=130), 1), (dict(E=9), 1),
    (dict(rows=-1), 1), (dict(dx="none"), 1), (dict(dx=(FAKE, None)), 1),
    (dict(dx=(FAKE, FAKE + 8)), 1), (dict(dw=(FAKE, FAKE + 2)), 1), (dict(x=None), 1),
    (dict(s2d=None), 1), (dict(x=FAKE + 8), 1), (dict(dw=(FAKE, FAKE), idx=None), 1),
    (dict(idx=FAKE + 4, dw=(FAKE, None)), 1), (dict(T=1 << 28, k=8), 2),
])
def test_dispatch_ranked_rejects(over, code):
    a = dict(x=FAKE, idx=FAKE, w=None, T=4, H=256, k=2, E=8, G=2, s2d=FAKE, dx=(FAKE, FAKE),
             dw=None, rows=16)
    a.update(over)
    dx = None if a["dx"] == "none" else _table(*a["dx"])
    dw = None if a["dw"] is None else _table(*a["dw"])
    keep = (dx, dw)
    st = ep.lib().ep_dispatch_ranked(a["x"], a["idx"], a["w"], a["T"], a["H"], a["k"], a["E"],
                                     a["G"], a["s2d"],
                                     None if dx is None else ctypes.addressof(dx),
                                     None if dw is None else ctypes.addressof(dw), a["rows"], None)
    del keep
    assert st == code, ep.last_error()
    assert ep.last_error()


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(G=0), 1), (dict(G=65), 1), (dict(H=20), 1), (dict(rows=-1), 1), (dict(T=-1), 1),
    (dict(src="none"), 1), (dict(src=(FAKE, None)), 1), (dict(src=(FAKE, FAKE + 4)), 1),
    (dict(s2d=None), 1), (dict(out=None), 1), (dict(out=FAKE + 8), 1),
    (dict(T=1 << 28, G=8, src=(FAKE,) * 8), 2),
])
def test_combine_ranked_rejects(over, code):
    a = dict(src=(FAKE, FAKE), rows=16, s2d=FAKE, T=4, H=256, G=2, out=FAKE)
    a.update(over)
    src = None if a["src"] == "none" else _table(*a["src"])
    st = ep.lib().ep_combine_ranked(None if src is None else ctypes.addressof(src), a["rows"],
                                    a["s2d"], a["T"], a["H"], a["G"], a["out"], None)
    assert st == code, ep.last_error()
    assert ep.last_error()


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(G=0), 1), (dict(G=65), 1), (dict(E=7), 1), (dict(rows=-1), 1), (dict(T=-1), 1),
    (dict(k=0), 1), (dict(gx="none", gw="none"), 1), (dict(out_x=None), 1), (dict(out_w=None), 1),
    (dict(gx=(FAKE, FAKE + 4)), 1), (dict(gx=(FAKE, None)), 1), (dict(H=20), 1),
    (dict(gw=(FAKE, FAKE + 2)), 1), (dict(idx=None), 1), (dict(idx=FAKE + 4), 1),
    (dict(out_x=FAKE + 8), 1), (dict(out_w=FAKE + 2), 1), (dict(s2d=None), 1),
    (dict(T=1 << 28, G=8, gx=(FAKE,) * 8, gw=(FAKE,) * 8), 2),
])
def test_dispatch_ranked_backward_rejects(over, code):
    a = dict(gx=(FAKE, FAKE), gw=(FAKE, FAKE), rows=16, idx=FAKE, s2d=FAKE, T=4, H=256, k=2, E=8,
             G=2, out_x=FAKE, out_w=FAKE)
    a.update(over)
    gx = None if a["gx"] == "none" else _table(*a["gx"])
    gw = None if a["gw"] == "none" else _table(*a["gw"])
    st = ep.lib().ep_dispatch_ranked_backward(
        None if gx is None else ctypes.addressof(gx), None if gw is None else ctypes.addressof(gw),
        a["rows"], a["idx"], a["s2d"], a["T"], a["H"], a["k"], a["E"], a["G"], a["out_x"],
        a["out_w"], None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def test_ranked_zero_tokens_are_noops():
    dx = _table(FAKE, FAKE)
    assert ep.lib().ep_dispatch_ranked(None, None, None, 0, 256, 2, 8, 2, None,
                                       ctypes.addressof(dx), None, 0, None) == 0
    assert ep.lib().ep_combine_ranked(ctypes.addressof(dx), 0, None, 0, 256, 2, None, None) == 0
    assert ep.lib().ep_routing_map(None, 0, 2, 8, None, None, None) == 0
    assert ep.lib().ep_dispatch_ranked_backward(ctypes.addressof(dx), ctypes.addressof(dx), 0, None,
                                                None, 0, 256, 2, 8, 2, FAKE, FAKE, None) == 0
    assert ep.last_error() == ""


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(G=0), 1), (dict(G=65, E=130), 1), (dict(E=9), 1), (dict(rank=2), 1),
    (dict(rank=-1), 1), (dict(H=12), 1), (dict(k=0), 1), (dict(rows=-1), 1), (dict(T=-1), 1),
    (dict(T=1 << 28, G=8, k=8, sx=(FAKE,) * 8), 2),
    (dict(sx="none"), 1), (dict(sx=(FAKE, None)), 1), (dict(sx=(FAKE, FAKE + 8)), 1),
    (dict(si="none"), 1), (dict(si=(FAKE, None)), 1), (dict(si=(FAKE, FAKE + 4)), 1),
    (dict(sw=(FAKE, FAKE + 2)), 1), (dict(src=None), 1), (dict(slot=None), 1),
    (dict(rti=None), 1), (dict(out=None), 1), (dict(out=FAKE + 8), 1), (dict(nr=FAKE + 2), 1),
])
def test_dispatch_fused_permute_rejects(over, code):
    a = dict(sx=(FAKE, FAKE), si=(FAKE, FAKE), sw=None, T=4, H=256, k=2, E=8, G=2, rank=0,
             src=FAKE, rti=FAKE, nr=None, slot=FAKE, rows=16, out=FAKE, rw=FAKE)
    a.update(over)
    tabs = {n: (None if a[n] in (None, "none") else _table(*a[n])) for n in ("sx", "si", "sw")}
    st = ep.lib().ep_dispatch_fused_permute(
        *[None if tabs[n] is None else ctypes.addressof(tabs[n]) for n in ("sx", "si", "sw")],
        a["T"], a["H"], a["k"], a["E"], a["G"], a["rank"], a["src"], a["rti"], a["nr"], a["slot"],
        a["rows"], a["out"], a["rw"], None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def test_dispatch_fused_permute_zero_tokens_is_a_noop():
    sx = _table(FAKE, FAKE)
    assert ep.lib().ep_dispatch_fused_permute(ctypes.addressof(sx), None, None, 0, 256, 2, 8, 2,
                                              0, None, None, None, None, 0, None, None, None) == 0
    assert ep.last_error() == ""


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(G=0), 1), (dict(E=9), 1), (dict(rank=2), 1), (dict(H=136), 1), (dict(H=8), 1),
    (dict(k=0), 1), (dict(rows=-1), 1), (dict(T=-1), 1),
    (dict(sq="none"), 1), (dict(sq=(FAKE, FAKE + 8)), 1), (dict(ss="none"), 1),
    (dict(ss=(FAKE, None)), 1), (dict(ss=(FAKE, FAKE + 2)), 1), (dict(si="none"), 1),
    (dict(sw=(FAKE, FAKE + 2)), 1), (dict(src=None), 1), (dict(slot=None), 1),
    (dict(out_q=None), 1), (dict(out_q=FAKE + 8), 1), (dict(out_s=None), 1),
    (dict(out_s=FAKE + 2), 1), (dict(nr=FAKE + 2), 1),
])
def test_dispatch_fused_permute_prequantized_rejects(over, code):
    a = dict(sq=(FAKE, FAKE), ss=(FAKE, FAKE), si=(FAKE, FAKE), sw=None, T=4, H=256, k=2, E=8,
             G=2, rank=0, src=FAKE, rti=FAKE, nr=None, slot=FAKE, rows=16, out_q=FAKE,
             out_s=FAKE, rw=FAKE)
    a.update(over)
    names = ("sq", "ss", "si", "sw")
    tabs = {n: (None if a[n] in (None, "none") else _table(*a[n])) for n in names}
    st = ep.lib().ep_dispatch_fused_permute_prequantized(
        *[None if tabs[n] is None else ctypes.addressof(tabs[n]) for n in names],
        a["T"], a["H"], a["k"], a["E"], a["G"], a["rank"], a["src"], a["rti"], a["nr"], a["slot"],
        a["rows"], a["out_q"], a["out_s"], a["rw"], None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def test_dispatch_fused_permute_prequantized_zero_tokens_is_a_noop():
    sq = _table(FAKE, FAKE)
    assert ep.lib().ep_dispatch_fused_permute_prequantized(
        ctypes.addressof(sq), ctypes.addressof(sq), None, None, 0, 256, 2, 8, 2, 0, None, None,
        None, None, 0, None, None, None, None) == 0
    assert ep.last_error() == ""


@no_gpu
@pytest.mark.parametrize("fmt,scale,ld,code", [
    (1, 0, 6, 1),      # fp32 scales: ld not a multiple of 4
    (1, 2, 20, 1),     # UE8M0: ld not a multiple of 16
    (1, 0, -4, 1),     # negative
    (0, 0, 16, 1),     # bf16 output takes no scale_ld
])
def test_dispatch_ex_rejects_scale_ld(fmt, scale, ld, code):
    st = ep.lib().ep_dispatch_ex(FAKE, 4, 256, 2, FAKE, None, fmt, scale, FAKE,
                                 FAKE if fmt else None, None, ld, None)
    assert st == code, ep.last_error()
    assert "scale_ld" in ep.last_error()


@no_gpu
def test_dispatch_prequantized_rejects_scale_ld():
    st = ep.lib().ep_dispatch_prequantized(FAKE, FAKE, 4, 256, 2, FAKE, None, FAKE, FAKE, None,
                                           6, None)
    assert st == 1 and "scale_ld" in ep.last_error()


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(H=200), 1), (dict(k=0), 1), (dict(G=65, E=130), 1), (dict(E=9), 1), (dict(rows=-1), 1),
    (dict(dq="none"), 1), (dict(ds="none"), 1), (dict(dq=(FAKE, FAKE + 8)), 1),
    (dict(ds=(FAKE, FAKE + 2)), 1), (dict(ds=(FAKE, None)), 1), (dict(dw=(FAKE, FAKE + 2)), 1),
    (dict(x=None), 1), (dict(xs=None), 1), (dict(s2d=None), 1), (dict(x=FAKE + 8), 1),
    (dict(xs=FAKE + 2), 1), (dict(dw=(FAKE, FAKE), idx=None), 1), (dict(T=1 << 28, k=8), 2),
])
def test_dispatch_ranked_prequantized_rejects(over, code):
    a = dict(x=FAKE, xs=FAKE, idx=FAKE, w=None, T=4, H=256, k=2, E=8, G=2, s2d=FAKE,
             dq=(FAKE, FAKE), ds=(FAKE, FAKE), dw=None, rows=16)
    a.update(over)
    tabs = {n: (None if a[n] in (None, "none") else _table(*a[n])) for n in ("dq", "ds", "dw")}
    st = ep.lib().ep_dispatch_ranked_prequantized(
        a["x"], a["xs"], a["idx"], a["w"], a["T"], a["H"], a["k"], a["E"], a["G"], a["s2d"],
        *[None if tabs[n] is None else ctypes.addressof(tabs[n]) for n in ("dq", "ds", "dw")],
        a["rows"], None)
    assert st == code, ep.last_error()
    assert ep.last_error()


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(fmt=0), 1), (dict(fmt=3), 1), (dict(sc=3), 1), (dict(H=200), 1), (dict(k=0), 1),
    (dict(G=65, E=130), 1), (dict(E=9), 1), (dict(rows=-1), 1), (dict(dq="none"), 1),
    (dict(ds="none"), 1), (dict(dq=(FAKE, FAKE + 8)), 1), (dict(ds=(FAKE, FAKE + 2)), 1),
    (dict(ds=(FAKE, None)), 1), (dict(dw=(FAKE, FAKE + 2)), 1), (dict(x=None), 1),
    (dict(s2d=None), 1), (dict(x=FAKE + 8), 1), (dict(dw=(FAKE, FAKE), idx=None), 1),
    (dict(T=1 << 28, k=8), 2),
    # 2^28 tokens of 7168 channels to 16 ranks: 7 tiles x 2 rank groups each
    (dict(T=1 << 28, k=1, H=7168, G=16, E=16, dq=(FAKE,) * 16, ds=(FAKE,) * 16), 2),
])
def test_dispatch_ranked_fp8_rejects(over, code):
    a = dict(x=FAKE, idx=FAKE, w=None, T=4, H=256, k=2, E=8, G=2, s2d=FAKE, fmt=1, sc=0,
             dq=(FAKE, FAKE), ds=(FAKE, FAKE), dw=None, rows=16)
    a.update(over)
    tabs = {n: (None if a[n] in (None, "none") else _table(*a[n])) for n in ("dq", "ds", "dw")}
    st = ep.lib().ep_dispatch_ranked_fp8(
        a["x"], a["idx"], a["w"], a["T"], a["H"], a["k"], a["E"], a["G"], a["s2d"], a["fmt"],
        a["sc"], *[None if tabs[n] is None else ctypes.addressof(tabs[n]) for n in ("dq", "ds", "dw")],
        a["rows"], None)
    assert st == code, ep.last_error()
    assert ep.last_error()


def test_dispatch_ranked_fp8_zero_tokens_is_a_noop():
    dq = _table(FAKE, FAKE)
    assert ep.lib().ep_dispatch_ranked_fp8(None, None, None, 0, 256, 2, 8, 2, None, 1, 2,
                                           ctypes.addressof(dq), ctypes.addressof(dq), None, 0,
                                           None) == 0
    assert ep.last_error() == ""


@no_gpu
def test_colmajor_workspace_size():
    lib = ep.lib()
    assert lib.ep_dispatch_colmajor_workspace_size(8192, 7168, 0) == 8192 * 56 * 4
    assert lib.ep_dispatch_colmajor_workspace_size(3, 256, 2) == 256   # 6 bytes, rounded up
    assert lib.ep_dispatch_colmajor_workspace_size(10, 200, 0) == 0    # not a multiple of 128
    assert lib.ep_dispatch_colmajor_workspace_size(10, 256, 7) == 0    # unknown scale format


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(fmt=0), 1), (dict(fmt=3), 1), (dict(scale=5), 1), (dict(H=200), 1), (dict(k=0), 1),
    (dict(T=-1), 1), (dict(ld=0), 1), (dict(ld=6), 1), (dict(scale=2, ld=20), 1),
    (dict(rows=-1), 1), (dict(rows=20), 1), (dict(rows=1 << 31, ld=1 << 32), 1),
    (dict(ws=None), 1), (dict(ws=FAKE + 16), 1), (dict(wsb=255), 1), (dict(x=None), 1),
    (dict(slot=None), 1), (dict(src=None), 1), (dict(q=None), 1), (dict(s=None), 1),
    (dict(x=FAKE + 8), 1), (dict(q=FAKE + 8), 1), (dict(s=FAKE + 2), 1), (dict(rw=FAKE), 1),
])
def test_dispatch_colmajor_scales_rejects(over, code):
    a = dict(x=FAKE, T=4, H=256, k=2, slot=FAKE, src=FAKE, w=None, fmt=1, scale=0, q=FAKE, s=FAKE,
             rw=None, ld=16, rows=8, ws=FAKE, wsb=256)
    a.update(over)
    st = ep.lib().ep_dispatch_colmajor_scales(
        a["x"], a["T"], a["H"], a["k"], a["slot"], a["src"], a["w"], a["fmt"], a["scale"], a["q"],
        a["s"], a["rw"], a["ld"], a["rows"], a["ws"], a["wsb"], None)
    assert st == code, ep.last_error()
    assert ep.last_error()


@no_gpu
def test_dispatch_colmajor_scales_zero_tokens_is_a_noop():
    st = ep.lib().ep_dispatch_colmajor_scales(None, 0, 256, 2, None, None, None, 1, 0, None, None,
                                              None, 16, 0, FAKE, 256, None)
    assert st == 0 and ep.last_error() == ""


@no_gpu
@pytest.mark.parametrize("over,code", [
    (dict(H=200), 1), (dict(k=0), 1), (dict(T=-1), 1), (dict(ld=0), 1), (dict(ld=6), 1),
    (dict(rows=-1), 1), (dict(rows=20), 1), (dict(rows=1 << 31, ld=1 << 32), 1),
    (dict(xq=None), 1), (dict(xs=None), 1), (dict(slot=None), 1), (dict(src=None), 1),
    (dict(q=None), 1), (dict(s=None), 1), (dict(xq=FAKE + 8), 1), (dict(q=FAKE + 8), 1),
    (dict(xs=FAKE + 2), 1), (dict(s=FAKE + 2), 1), (dict(rw=FAKE), 1),
])
def test_dispatch_prequantized_colmajor_rejects(over, code):
    a = dict(xq=FAKE, xs=FAKE, T=4, H=256, k=2, slot=FAKE, src=FAKE, w=None, q=FAKE, s=FAKE,
             rw=None, ld=16, rows=8)
    a.update(over)
    st = ep.lib().ep_dispatch_prequantized_colmajor(
        a["xq"], a["xs"], a["T"], a["H"], a["k"], a["slot"], a["src"], a["w"], a["q"], a["s"],
        a["rw"], a["ld"], a["rows"], None)
    assert st == code, ep.last_error()
    assert ep.last_error()


@no_gpu
def test_dispatch_prequantized_colmajor_zero_tokens_is_a_noop():
    st = ep.lib().ep_dispatch_prequantized_colmajor(None, None, 0, 256, 2, None, None, None, None,
                                                    None, None, 16, 0, None)
    assert st == 0 and ep.last_error() == ""
