"""Time the bf16 dispatch next to kernels that isolate its access pattern,
on the headline workload (T=8192, hidden 7168, E=256, k=8), caches emptied
(1 GiB read) before every launch, HIP events on the launch stream.

    python -m combine_ep_layout_04_amd.probes.write_pattern [--rounds 6] [--reps 20]
    python -m combine_ep_layout_04_amd.probes.write_pattern --pmc   # 3 launches each, for rocprofv3 --pmc

Kernels: the library's ep_dispatch; stores_only (its grid, XCD order and
slot map, no loads of x); write streams of the same bytes in destination
order (2 KiB and 4 KiB one-shot workgroups, 14 KiB per workgroup in turn);
a read of x; the dispatch in destination order (gather: x read k times);
the stores-only grid under other slot maps (each token's rows adjacent, k
sequential streams, a random permutation); whole rows copied in token
order, destination order, or windows of 256 tokens expert by expert, and
in windows of 64 tokens expert by expert with each window on one XCD; and
for the 8-bit cast, the library's E4M3 dispatch next to the same slot
map stored at its code-row size and a stream of its code bytes."""

import argparse
import ctypes
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
PROBE_LIB = os.path.join(HERE, "libep_probe.so")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--rounds", type=int, default=6)
    ap.add_argument("--pmc", action="store_true")
    args = ap.parse_args()

    import numpy as np
    import torch

    from combine_ep_layout_04_amd import ep
    from combine_ep_layout_04_amd.inputs import WORKLOADS, make_inputs

    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing; build it with `python -m combine_ep_layout_04_amd.build`")
    L = ep.lib()
    pr = ctypes.CDLL(PROBE_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    pr.probe_stores_only.argtypes = [i64, i32, i32, vp, vp, vp]
    pr.probe_write_stream.argtypes = [vp, i64, i32, vp]
    pr.probe_read_x.argtypes = [vp, i64, vp, vp]
    pr.probe_gather.argtypes = [vp, i32, i32, vp, vp, vp]
    pr.probe_order_rows.argtypes = [vp, i64, i32, i32, vp, i32, vp, vp, vp]

    w = WORKLOADS["headline"]
    inp = make_inputs(w)
    T, H, E, k = w.T, w.H, w.E, w.k
    P = T * k
    dev = torch.device("cuda:0")
    st = torch.cuda.Stream(device=dev)
    s = st.cuda_stream
    i32d = dict(dtype=torch.int32, device=dev)
    with torch.cuda.stream(st):
        idx = torch.from_numpy(inp.topk_idx).to(dev)
        x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        counts, offsets = torch.empty(E, **i32d), torch.empty(E + 1, **i32d)
        slot, src = torch.empty((T, k), **i32d), torch.empty(P, **i32d)
        wsb = ep.layout_workspace_size(T, k, E)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        recv = torch.empty((P, H), dtype=torch.bfloat16, device=dev)
        q8 = torch.empty((P, H), dtype=torch.uint8, device=dev)
        s8 = torch.empty((P, H // 128), dtype=torch.float32, device=dev)
        sink = torch.zeros(4, **i32d)
        scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    st.synchronize()
    if L.ep_layout(idx.data_ptr(), T, k, E, counts.data_ptr(), offsets.data_ptr(), slot.data_ptr(),
                   src.data_ptr(), None, ws.data_ptr(), wsb, s) != 0:
        raise SystemExit("ep_layout failed")
    st.synchronize()
    n = int(offsets[E].item())
    if n != P:
        raise SystemExit("the probes assume no masked slots")
    wbytes = n * H * 2
    # other slot maps for the stores-only grid, and visiting orders of the
    # receive rows (permutations of [0, P)) for the whole-row copy
    slot_h = slot.cpu().numpy()
    tok = np.repeat(np.arange(T), k)
    rows = slot_h.reshape(-1)
    perm = np.random.default_rng(0).permutation(P)
    orders = {
        "token order": rows,
        "destination order": np.arange(P),
        "windows of 256 tokens, expert by expert": rows[np.lexsort((tok, inp.topk_idx.reshape(-1),
                                                                    tok // 256))],
    }
    # windows of 64 tokens, each on one XCD (window w on XCD w mod 8), its
    # rows expert by expert: 8 lists padded with -1
    ex = inp.topk_idx.reshape(-1)
    lists = [[] for _ in range(8)]
    for w0 in range(0, T, 64):
        sel = np.nonzero((tok >= w0) & (tok < w0 + 64))[0]
        lists[(w0 // 64) % 8].append(rows[sel[np.lexsort((tok[sel], ex[sel]))]])
    lists = [np.concatenate(li) for li in lists]
    per_xcd = max(len(li) for li in lists)
    xcd_lists = np.full((8, per_xcd), -1, np.int32)
    for i, li in enumerate(lists):
        xcd_lists[i, :len(li)] = li
    with torch.cuda.stream(st):
        d_xcd_lists = torch.from_numpy(xcd_lists).to(dev)
        maps = {"each token's rows adjacent (t*k+j)": torch.arange(P, **i32d).view(T, k),
                "k sequential streams (j*T+t)": torch.arange(P, **i32d).view(k, T).t().contiguous(),
                "a random permutation": torch.from_numpy(perm.astype(np.int32)).to(dev).view(T, k)}
        d_orders = {nm: torch.from_numpy(np.ascontiguousarray(o, dtype=np.int32)).to(dev)
                    for nm, o in orders.items()}
    st.synchronize()
    ops = {
        "dispatch (library)": lambda: L.ep_dispatch(x.data_ptr(), T, H, k, slot.data_ptr(), None, 0,
                                                    recv.data_ptr(), None, None, s),
        "stores_only (same grid and slot map)": lambda: pr.probe_stores_only(T, H, k, slot.data_ptr(),
                                                                             recv.data_ptr(), s),
        "write stream, 2 KiB workgroups": lambda: pr.probe_write_stream(recv.data_ptr(), wbytes, 2, s),
        "write stream, 4 KiB workgroups": lambda: pr.probe_write_stream(recv.data_ptr(), wbytes, 4, s),
        "write stream, 14 KiB per workgroup": lambda: pr.probe_write_stream(recv.data_ptr(), wbytes, 14, s),
        "read x": lambda: pr.probe_read_x(x.data_ptr(), T * H * 2, sink.data_ptr(), s),
        "gather (destination order)": lambda: pr.probe_gather(x.data_ptr(), H, n, src.data_ptr(),
                                                              recv.data_ptr(), s),
        **{f"stores_only, slot map: {nm}": (lambda m=m: pr.probe_stores_only(T, H, k, m.data_ptr(),
                                                                              recv.data_ptr(), s))
           for nm, m in maps.items()},
        **{f"whole rows in {nm}": (lambda o=o: pr.probe_order_rows(x.data_ptr(), T, H, n, o.data_ptr(), 0,
                                                                  src.data_ptr(), recv.data_ptr(), s))
           for nm, o in d_orders.items()},
        "whole rows in windows of 64 tokens on one XCD each, expert by expert": lambda: pr.probe_order_rows(
            x.data_ptr(), T, H, n, d_xcd_lists.data_ptr(), per_xcd, src.data_ptr(), recv.data_ptr(), s),
        # the 8-bit cast writes rows of H code bytes (and H/128 scales): the
        # same slot map stored at that row size, with no loads
        "fp8 dispatch (library, E4M3, fp32 scales)": lambda: L.ep_dispatch(
            x.data_ptr(), T, H, k, slot.data_ptr(), None, 1, q8.data_ptr(), s8.data_ptr(), None, s),
        "stores_only at the fp8 code row size": lambda: pr.probe_stores_only(T, H // 2, k, slot.data_ptr(),
                                                                             q8.data_ptr(), s),
        "write stream of the fp8 code bytes, 2 KiB workgroups": lambda: pr.probe_write_stream(
            q8.data_ptr(), n * H, 2, s),
    }
    algo = {"dispatch (library)": T * H * 2 + wbytes + P * 4, "read x": T * H * 2,
            "gather (destination order)": T * H * 2 + wbytes + P * 4,
            **{f"whole rows in {nm}": T * H * 2 + wbytes + P * 4 for nm in orders},
            "whole rows in windows of 64 tokens on one XCD each, expert by expert": T * H * 2 + wbytes + P * 4,
            "fp8 dispatch (library, E4M3, fp32 scales)": T * H * 2 + n * H + n * (H // 128) * 4 + P * 4,
            "stores_only at the fp8 code row size": n * H,
            "write stream of the fp8 code bytes, 2 KiB workgroups": n * H}

    def flush():
        with torch.cuda.stream(st):
            scratch.sum()

    def call(name, fn):
        rc = fn()
        if rc != 0:
            raise SystemExit(f"{name}: status {rc}")

    if args.pmc:
        for name, fn in ops.items():
            for _ in range(3):
                flush()
                call(name, fn)
            st.synchronize()
            print(f"[write_pattern] {name}: 3 launches", flush=True)
        return

    def time_fn(name, fn):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.reps)]
        for i in range(-2, args.reps):
            flush()
            if i >= 0:
                ev[i][0].record(st)
            call(name, fn)
            if i >= 0:
                ev[i][1].record(st)
        st.synchronize()
        return statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)

    res = {name: [] for name in ops}
    for r in range(args.rounds):
        for name, fn in ops.items():
            res[name].append(time_fn(name, fn))
        print(f"[write_pattern] round {r + 1}/{args.rounds}", flush=True)
    for name, v in res.items():
        m = statistics.median(v)
        b = algo.get(name, wbytes)
        print(f"[write_pattern] {name}: {m:.1f} us (rounds {min(v):.1f}-{max(v):.1f}), "
              f"{b / m / 1e3:.0f} GB/s of {b} B", flush=True)


if __name__ == "__main__":
    main()
