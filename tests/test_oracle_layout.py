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
    idx = np.array(case["topk_idx"], np.int64).reshape(T, k)
    L = oracle.layout(idx, E)
    np.testing.assert_array_equal(L.counts, case["counts"])
    np.testing.assert_array_equal(L.offsets, case["offsets"])
    np.testing.assert_array_equal(L.slot.reshape(-1), case["slot"])
    n = L.n
    np.testing.assert_array_equal(L.src[:n], case.get("src", []))
    assert L.num_invalid == case["invalid"][0]


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
    counts, offsets, slot, src, bad = brute.layout(inp.topk_idx, 8)
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
    counts, offsets, slot, src, bad = brute.layout(inp.topk_idx, E)
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
