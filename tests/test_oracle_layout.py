"""Pins for the oracle's layout (counts, exclusive offsets, stable slots, src).

Independent routes to the same answer:
* hand-worked fixtures (tests/golden/layout_handworked.txt);
* a library special case: numpy's stable argsort of the expert keys with
  masked pairs sorted last, bincount and cumsum;
* the pure-Python definition (oracle/brute.py) on tiny inputs;
* invariants any correct layout satisfies.
"""

import numpy as np
import pytest

import oracle
from oracle import brute
from combine_ep_layout_04_amd.inputs import WORKLOADS, make_inputs, make_random_case

from golden_io import read_cases


def numpy_layout(idx: np.ndarray, E: int):
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")
    n = int(valid.sum())
    slot = np.full(flat.shape, -1, np.int64)
    slot[order[:n]] = np.arange(n)
    counts = np.bincount(flat[valid], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    src = np.full(flat.shape, -1, np.int64)
    src[:n] = order[:n] // idx.shape[1]
    return counts, offsets, slot.reshape(idx.shape), src


def check_invariants(idx, E, L):
    T, k = idx.shape
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    n = int(valid.sum())
    assert L.counts.sum() == n == L.offsets[-1]
    assert L.offsets[0] == 0 and np.all(np.diff(L.offsets) == L.counts)
    s = L.slot.reshape(-1)
    assert np.all(s[~valid] == -1)
    # bijection of unmasked pairs onto [0, N)
    assert np.array_equal(np.sort(s[valid]), np.arange(n))
    # each expert's rows lie in its segment and rise with the flat index
    for e in np.unique(flat[valid]):
        rows = s[flat == e]
        assert rows.min() == L.offsets[e] and rows.max() == L.offsets[e + 1] - 1
        assert np.all(np.diff(rows) == 1)
    # src points back at the owning token
    t_of_pair = np.repeat(np.arange(T), k)
    assert np.array_equal(L.src[s[valid]], t_of_pair[valid])
    assert np.all(L.src[n:] == -1)
    bad = ~valid & (flat != -1)
    assert L.num_invalid == int(bad.sum())


@pytest.mark.parametrize("case", read_cases("layout_handworked.txt"), ids=lambda c: c["name"])
def test_layout_handworked(case):
    T, k, E = case["T"][0], case["k"][0], case["E"][0]
    A = case.get("alignment", [1])[0]
    cap = case.get("capacity", [0])[0]
    idx = np.array(case["topk_idx"], np.int64).reshape(T, k)
    L = oracle.layout(idx, E, alignment=A, capacity=cap)
    np.testing.assert_array_equal(L.counts, case["counts"])
    np.testing.assert_array_equal(L.offsets, case["offsets"])
    np.testing.assert_array_equal(L.slot.reshape(-1), case["slot"])
    n = L.n
    if "src_full" in case:
        np.testing.assert_array_equal(L.src[:n], case["src_full"])
    else:
        np.testing.assert_array_equal(L.src[:n], case.get("src", []))
    assert L.num_invalid == case["invalid"][0]
    assert L.num_dropped == case.get("dropped", [0])[0]


@pytest.mark.parametrize("name", ["tiny", "mid", "headline", "skewed", "fp8"])
def test_layout_workloads_vs_numpy_argsort(name):
    inp = make_inputs(WORKLOADS[name])
    E = WORKLOADS[name].E
    L = oracle.layout(inp.topk_idx, E)
    counts, offsets, slot, src = numpy_layout(inp.topk_idx, E)
    np.testing.assert_array_equal(L.counts, counts)
    np.testing.assert_array_equal(L.offsets, offsets)
    np.testing.assert_array_equal(L.slot, slot)
    np.testing.assert_array_equal(L.src, src)
    check_invariants(inp.topk_idx, E, L)


def test_layout_tiny_vs_bruteforce():
    inp = make_inputs(WORKLOADS["tiny"])
    L = oracle.layout(inp.topk_idx, 8)
    counts, offsets, slot, src, bad, _ = brute.layout(inp.topk_idx, 8)
    np.testing.assert_array_equal(L.counts, counts)
    np.testing.assert_array_equal(L.offsets, offsets)
    np.testing.assert_array_equal(L.slot, slot)
    np.testing.assert_array_equal(L.src, src)
    assert L.num_invalid == bad == 0


@pytest.mark.parametrize("seed", range(200))
def test_layout_random_tiny_vs_bruteforce(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(1, 33))
    k = int(rng.integers(1, 5))
    E = int(rng.integers(1, 17))
    inp = make_random_case(seed, T, 8, E, k, mask_frac=float(rng.uniform(0, 0.5)),
                           dup_frac=1.0, invalid_frac=float(rng.uniform(0, 0.2)))
    L = oracle.layout(inp.topk_idx, E)
    counts, offsets, slot, src, bad, _ = brute.layout(inp.topk_idx, E)
    np.testing.assert_array_equal(L.counts, counts)
    np.testing.assert_array_equal(L.offsets, offsets)
    np.testing.assert_array_equal(L.slot, slot)
    np.testing.assert_array_equal(L.src, src)
    assert L.num_invalid == bad
    check_invariants(inp.topk_idx, E, L)


def test_layout_workload_statistics():
    # the recipes produce what they promise: distinct experts per row for
    # the uniform workloads, exactly 5 % masked slots for the skewed one,
    # and a heavier head under the Zipf popularity
    for name in ("tiny", "mid", "headline", "fp8"):
        inp = make_inputs(WORKLOADS[name])
        s = np.sort(inp.topk_idx, axis=1)
        assert np.all(np.diff(s, axis=1) > 0)
    sk = make_inputs(WORKLOADS["skewed"])
    assert int((sk.topk_idx == -1).sum()) == round(0.05 * 8192 * 8)
    unm = sk.topk_idx[sk.topk_idx >= 0]
    c = np.bincount(unm, minlength=256)
    assert c.max() > 8 * c.mean()


# ------------------------------------------------ aligned and fixed-stride --

def numpy_layout_ex(idx: np.ndarray, E: int, A: int, cap: int):
    """Library special case: stable argsort ranks, placed by segment start."""
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")
    raw = np.bincount(flat[valid], minlength=E)
    first = np.concatenate([[0], np.cumsum(raw)])
    rank = np.empty(flat.shape, np.int64)
    rank[order] = np.arange(flat.size) - first[key[order]]
    if cap > 0:
        start = np.arange(E) * cap
        keep = valid & (rank < cap)
    else:
        padded = -(-raw // A) * A
        start = np.concatenate([[0], np.cumsum(padded)])[:E]
        keep = valid
    slot = np.where(keep, start[np.where(valid, flat, 0)] + rank, -1)
    return slot.reshape(idx.shape), int((valid & ~keep).sum())


@pytest.mark.parametrize("A,cap", [(1, 0), (4, 0), (128, 0), (1, 64), (8, 64), (1, 256)])
@pytest.mark.parametrize("name", ["tiny", "mid", "skewed"])
def test_layout_ex_workloads(name, A, cap):
    w = WORKLOADS[name]
    inp = make_inputs(w, T=min(w.T, 2048))
    E = w.E
    L = oracle.layout(inp.topk_idx, E, alignment=A, capacity=cap)
    slot, dropped = numpy_layout_ex(inp.topk_idx, E, A, cap)
    np.testing.assert_array_equal(L.slot, slot)
    assert L.num_dropped == dropped
    flat = inp.topk_idx.reshape(-1)
    raw = np.bincount(flat[flat >= 0], minlength=E)
    if cap > 0:
        np.testing.assert_array_equal(L.counts, np.minimum(raw, cap))
        np.testing.assert_array_equal(L.offsets, np.arange(E + 1) * cap)
        assert dropped == int(np.maximum(raw - cap, 0).sum())
    else:
        # the DeepEP expand-mode reading of the prefix sums: psum[i] is the
        # end of expert i's rows and the next start is align(psum[i], A)
        psum = L.offsets[:E] + L.counts
        np.testing.assert_array_equal(L.counts, raw)
        assert L.offsets[0] == 0
        np.testing.assert_array_equal(L.offsets[1:], -(-psum // A) * A)
    # every placed row belongs to its expert's segment and src points back
    s = L.slot.reshape(-1)
    t_of_pair = np.repeat(np.arange(inp.topk_idx.shape[0]), inp.topk_idx.shape[1])
    placed = s >= 0
    e = flat[placed]
    assert np.all(s[placed] >= L.offsets[e]) and np.all(s[placed] < L.offsets[e] + L.counts[e])
    np.testing.assert_array_equal(L.src[s[placed]], t_of_pair[placed])
    assert L.n <= oracle.max_rows(*inp.topk_idx.shape, E, A, cap)


@pytest.mark.parametrize("seed", range(120))
def test_layout_ex_random_tiny_vs_bruteforce(seed):
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.integers(1, 25))
    k = int(rng.integers(1, 4))
    E = int(rng.integers(1, 9))
    A = int(rng.choice([1, 2, 3, 4, 8]))
    cap = int(rng.choice([0, 0, 1, 2, 5])) * A
    inp = make_random_case(seed, T, 8, E, k, mask_frac=0.2, dup_frac=1.0, invalid_frac=0.1)
    L = oracle.layout(inp.topk_idx, E, alignment=A, capacity=cap)
    counts, offsets, slot, src, bad, dropped = brute.layout(inp.topk_idx, E, A, cap)
    np.testing.assert_array_equal(L.counts, counts)
    np.testing.assert_array_equal(L.offsets, offsets)
    np.testing.assert_array_equal(L.slot, slot)
    np.testing.assert_array_equal(L.src[:L.n], src[:L.n])
    assert L.num_invalid == bad and L.num_dropped == dropped
