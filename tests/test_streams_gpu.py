"""Concurrent calls: apart from the no-allocation layout's scratch, which
these pipelines do not use, the library keeps no state between calls (the
layout arrays and the caller's workspace are the only memory it touches),
so independent pipelines on different streams can overlap.

Two forward steps (layout -> bf16 and 8-bit dispatch, the 8-bit cast with
column-major scales through each pipeline's own workspace -> combine) with
different inputs and shapes are launched interleaved on two streams,
several rounds, with no synchronisation between the streams; every output
must equal the one from running the same pipeline alone on the default
stream, bit for bit (every kernel is deterministic).
"""

import numpy as np
import pytest
import torch

from combine_ep_layout_04_amd import ep
from combine_ep_layout_04_amd.inputs import make_random_case

from gpu_util import DEV, dev, x_dev

pytestmark = pytest.mark.gpu


class Pipeline:
    def __init__(self, seed, T, H, E, k):
        inp = make_random_case(seed, T, H, E, k, mask_frac=0.05, invalid_frac=0.01)
        self.E = E
        self.idx, self.x, self.w = dev(inp.topk_idx), x_dev(inp.x_bits), dev(inp.topk_weights)
        P = T * k
        i32 = dict(dtype=torch.int32, device=DEV)
        self.o = {
            "counts": torch.empty(E, **i32), "offsets": torch.empty(E + 1, **i32),
            "slot": torch.empty((T, k), **i32), "src": torch.empty(P, **i32),
            "inval": torch.empty(1, **i32),
            "recv": torch.empty((P, H), dtype=torch.bfloat16, device=DEV),
            "rw": torch.empty(P, dtype=torch.float32, device=DEV),
            "q": torch.empty((P, H), dtype=torch.uint8, device=DEV),
            "s": torch.empty((P, H // 128), dtype=torch.float32, device=DEV),
            "out": torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
            "q2": torch.empty((P, H), dtype=torch.uint8, device=DEV),
            "s2": torch.empty((H // 128, P + 16), dtype=torch.float32, device=DEV),
        }
        self.ld = P + 16
        self.cm_ws = torch.empty(max(ep.ep_dispatch_colmajor_workspace_size(T, H), 256),
                                 dtype=torch.uint8, device=DEV)
        self.ws = torch.empty(max(ep.layout_workspace_size(T, k, E), 256), dtype=torch.uint8,
                              device=DEV)

    def reset(self):
        for t in self.o.values():
            t.view(torch.uint8).fill_(0x55)

    def steps(self, stream):
        """The pipeline as a list of launches (so two can be interleaved)."""
        o = self.o
        return [
            lambda: ep.ep_layout(self.idx, self.E, counts=o["counts"], offsets=o["offsets"],
                                 slot=o["slot"], src=o["src"], num_invalid=o["inval"],
                                 workspace=self.ws, stream=stream),
            lambda: ep.ep_dispatch(self.x, o["slot"], self.w, recv_x=o["recv"], recv_weights=o["rw"],
                                   stream=stream),
            lambda: ep.ep_dispatch(self.x, o["slot"], None, fp8=True, recv_x=o["q"],
                                   recv_scales=o["s"], stream=stream),
            lambda: ep.ep_dispatch_colmajor_scales(self.x, o["slot"], o["src"], None,
                                                   scale_ld=self.ld, recv_x=o["q2"],
                                                   recv_scales=o["s2"], workspace=self.cm_ws,
                                                   stream=stream),
            lambda: ep.ep_combine(o["recv"], o["slot"], self.w, out=o["out"], stream=stream),
        ]

    def snapshot(self):
        return {n: t.clone() for n, t in self.o.items()}


def test_two_pipelines_on_two_streams():
    a = Pipeline(81, 2048, 7168, 64, 8)     # tiled kernels
    b = Pipeline(82, 3000, 1536, 40, 6)     # narrow tiles, per-token dispatch
    print("\n[streams] two pipelines, interleaved on two streams", flush=True)
    refs = []
    for p in (a, b):
        p.reset()
        torch.cuda.synchronize()
        for f in p.steps(None):
            f()
        torch.cuda.synchronize()
        refs.append(p.snapshot())
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rnd in range(3):
        for p in (a, b):
            p.reset()
        torch.cuda.synchronize()
        for fa, fb in zip(a.steps(sa), b.steps(sb)):
            fa()
            fb()
        torch.cuda.synchronize()
        for p, ref in zip((a, b), refs):
            for n, t in p.o.items():
                assert torch.equal(t.view(torch.uint8), ref[n].view(torch.uint8)), f"round {rnd}: {n}"
