"""Pins for the oracle's top-k routing, softmax over the selected logits, and binning.

Pinned against a brute-force Python implementation (sorted(), explicit loops),
invariants of the counting sort and m-tile walk (sum of counts = n*k, each pair once,
tiles = sum_e ceil(count_e / tile_m), from the gate-the-grouped-GEMM page, PR #167,
"The cause is a threshold"), and closed-form special cases.
"""
import math

import numpy as np
import pytest

from oracle import routing


@pytest.mark.parametrize("seed,n,E,k", [(0, 37, 8, 2), (1, 64, 16, 4), (2, 50, 256, 6), (3, 5, 6, 6)])
def test_route_matches_bruteforce_with_ties(seed, n, E, k):
    rng = np.random.default_rng(seed)
    logits = np.round(rng.standard_normal((n, E)) * 2).astype(np.float32)   # many exact ties
    logits[0, :] = 0.0
    logits[1 % n, :] = -0.0
    i1, w1 = routing.route_topk(logits, k)
    i2, w2 = routing.route_topk_bruteforce(logits, k)
    assert np.array_equal(i1, i2)
    assert np.allclose(w1, w2, rtol=2e-7, atol=0)
    assert np.array_equal(i1[0], np.arange(k))       # all-equal row: lowest indices, in order


def test_route_descending_and_distinct():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((100, 256)).astype(np.float32)
    idx, w = routing.route_topk(logits, 6)
    sel = np.take_along_axis(logits, idx, axis=1)
    assert np.all(np.diff(sel, axis=1) <= 0)
    assert all(len(set(r)) == 6 for r in idx.tolist())
    # every unselected logit is <= the smallest selected one
    for t in range(100):
        rest = np.delete(logits[t], idx[t])
        assert rest.max() <= sel[t, -1]
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_k_equals_E_equal_logits_gives_uniform_weights():
    idx, w = routing.route_topk(np.full((3, 5), 1.25, np.float32), 5)
    assert np.array_equal(idx, np.tile(np.arange(5), (3, 1)))
    assert np.allclose(w, 0.2, rtol=0, atol=1e-7)


def test_softmax_closed_form_two_experts():
    idx, w = routing.route_topk(np.array([[0.0, math.log(3.0), -5.0]], np.float32), 2)
    assert idx.tolist() == [[1, 0]]
    assert w[0].tolist() == pytest.approx([0.75, 0.25], rel=1e-6)


@pytest.mark.parametrize("seed,n,E,k,tm", [(0, 16, 8, 2, 16), (1, 100, 16, 4, 16), (2, 257, 64, 6, 16),
                                          (3, 400, 32, 3, 7), (4, 1, 8, 8, 16)])
def test_bin_matches_bruteforce_and_invariants(seed, n, E, k, tm):
    rng = np.random.default_rng(seed)
    idx, _ = routing.route_topk(rng.standard_normal((n, E)).astype(np.float32), k)
    a = routing.bin_pairs(idx, E, tm)
    b = routing.bin_pairs_bruteforce(idx, E, tm)
    for key in ("counts", "offsets", "sorted_pair", "tile_map"):
        assert np.array_equal(a[key], b[key]), key
    assert a["n_tiles"] == b["n_tiles"]
    assert a["counts"].sum() == n * k
    assert sorted(a["sorted_pair"].tolist()) == list(range(n * k))
    assert a["n_tiles"] == sum(math.ceil(c / tm) for c in a["counts"].tolist())
    flat = idx.reshape(-1)
    for e in range(E):
        seg = a["sorted_pair"][a["offsets"][e]:a["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)          # stable: ascending pair id
    tm_ = a["tile_map"]
    assert np.all(tm_[:, 2] >= 1) and np.all(tm_[:, 2] <= tm)
    assert np.all(np.diff(tm_[:, 0]) >= 0)
    # tiles tile each bin exactly
    for e in range(E):
        t = tm_[tm_[:, 0] == e]
        assert t[:, 2].sum() == a["counts"][e]
        if len(t):
            assert t[0, 1] == a["offsets"][e]
            assert np.all(t[1:, 1] == t[:-1, 1] + t[:-1, 2])
