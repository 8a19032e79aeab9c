"""Pins for the closed-form fill model and the grouped-arm predicate.

Pinned against the numbers printed on the gate-the-grouped-GEMM page (PR #167):
the fill table, the engagement log line, the post-merge arithmetic and the test
descriptions (tests/golden/fill_table.txt cites each section), plus exact
flip-point checks and the binomial expectation of the tile count.
"""
import math

import numpy as np
import pytest

from golden_io import records
from oracle import fill, routing


def _recs(kind):
    return [r[1:] for r in records("fill_table.txt") if r[0] == kind]


@pytest.mark.parametrize("rec", _recs("table"))
def test_fill_table_printed_digits(rec):
    n, pairs, woken, ppe, fillpct = int(rec[0]), int(rec[1]), rec[2], rec[3], rec[4]
    assert n * 6 == pairs
    assert f"{fill.woken_experts(n, 6, 256):.1f}" == woken
    assert f"{fill.pairs_per_woken_expert(n, 6, 256):.{len(ppe.split('.')[1])}f}" == ppe
    assert f"{100 * fill.tile_fill(n, 6, 256, 16):.1f}" == fillpct


def test_engagement_line():
    (n, k, E, tm, pct, ppe, boundary), = _recs("engaged")
    n, k, E, tm = int(n), int(k), int(E), int(tm)
    assert f"{fill.pairs_per_woken_expert(n, k, E):.2f}" == ppe
    assert f"{100 * fill.tile_fill(n, k, E, tm):.0f}" == pct
    assert fill.min_tokens_grouped(k, E, tm) == int(boundary)
    assert fill.select_grouped(n, k, E, tm)


def test_postmerge_numbers():
    (n, k, E, v), = _recs("ppe")
    assert f"{fill.pairs_per_woken_expert(int(n), int(k), int(E)):.1f}" == v
    (k, E, tm, v), = _recs("min_tokens")
    assert fill.min_tokens_grouped(int(k), int(E), int(tm)) == int(v)


def test_selection_ranges_from_the_tests_section():
    (lo, hi, k, E, tm), = _recs("reject_range")
    for n in range(int(lo), int(hi) + 1):
        assert not fill.select_grouped(n, int(k), int(E), int(tm))
    (lo, k, E, tm), = _recs("accept_from")
    for n in range(int(lo), int(lo) + 400):
        assert fill.select_grouped(n, int(k), int(E), int(tm))
    (n, k, E, tm), = _recs("accept")
    assert fill.pairs_per_woken_expert(int(n), int(k), int(E)) == pytest.approx(24.0, abs=1e-9)
    assert fill.select_grouped(int(n), int(k), int(E), int(tm))


def test_decode_floor_and_ratio_at_flip():
    # n <= 8 never selects, whatever the routing shape
    for n in range(1, 9):
        assert not fill.select_grouped(n, 8, 8, 1)
    assert fill.pairs_per_woken_expert(682, 6, 256) < 16 <= fill.pairs_per_woken_expert(683, 6, 256)


SHAPES = [(k, E, tm) for (k, E) in [(1, 4), (2, 8), (4, 16), (6, 64), (6, 256), (8, 256), (2, 64),
                                      (8, 128), (1, 256), (6, 8)] for tm in (16, 32, 64)]


@pytest.mark.parametrize("k,E,tm", SHAPES)
def test_min_tokens_is_the_exact_flip_point(k, E, tm):
    n0 = fill.min_tokens_grouped(k, E, tm)
    assert fill.select_grouped(n0, k, E, tm)
    assert not fill.select_grouped(n0 - 1, k, E, tm)


def test_ppe_monotone_and_limits():
    prev = 0.0
    for n in range(1, 3000):
        v = fill.pairs_per_woken_expert(n, 6, 256)
        assert v >= prev - 1e-12
        prev = v
    assert fill.pairs_per_woken_expert(1, 6, 256) == pytest.approx(1.0)
    assert fill.pairs_per_woken_expert(10, 4, 4) == pytest.approx(10.0)   # k == E: every expert woken


def test_expected_tiles_against_simulation():
    rng = np.random.default_rng(0)
    n, k, E, tm = 200, 6, 64, 16
    sims = []
    for _ in range(300):
        idx = np.argsort(rng.random((n, E)), axis=1)[:, :k]
        b = routing.bin_pairs(idx, E, tm)
        sims.append(b["n_tiles"])
    assert fill.expected_tiles(n, k, E, tm) == pytest.approx(np.mean(sims), rel=0.01)


def test_expected_tiles_v4_values():
    # E[tiles] at tile_m = 16: the binomial spread makes mean occupancy well below the mean fill
    assert fill.expected_tiles(683, 6, 256, 16) == pytest.approx(367.3, abs=0.1)
    assert fill.expected_tiles(1024, 6, 256, 16) == pytest.approx(509.6, abs=0.1)
    # one tile per woken expert while no expert can reach a second tile
    assert fill.expected_tiles(10, 6, 256, 16) == pytest.approx(fill.woken_experts(10, 6, 256), rel=1e-9)


@pytest.mark.parametrize("k,E", [(k, E) for (k, E, tm) in SHAPES if tm == 16])
def test_equal_constants_leave_no_dequantize_window(k, E):
    # the Tests section: both boundary constants at 16 leave no n for the third arm
    n_max = fill.min_tokens_grouped(k, E, 16) + 200
    assert fill.dequant_tokens(k, E, 16, 16, n_max) == []
    # and a grouped threshold at or below the traffic ratio keeps it closed as well
    assert fill.dequant_tokens(k, E, 1, 16, n_max) == []


@pytest.mark.parametrize("k,E", [(6, 256), (2, 8), (8, 128)])
def test_a_higher_grouped_threshold_opens_the_window_exactly_between_the_flips(k, E):
    # grouped threshold 32 with traffic ratio 16: the dequantize arm takes exactly the n with
    # 16 <= pairs per woken expert < 32 above the decode floor, i.e. [min_tokens(16), min_tokens(32))
    lo, hi = fill.min_tokens_grouped(k, E, 16), fill.min_tokens_grouped(k, E, 32)
    got = fill.dequant_tokens(k, E, 32, 16, hi + 50)
    assert got == list(range(lo, hi))
    assert fill.select_arm(lo - 1, k, E, 32, 16) == "gemv"
    assert fill.select_arm(hi, k, E, 32, 16) == "grouped"


def test_three_arm_dispatch_v4_values():
    # V4 (top-6 of 256): the fused GEMV below 683 tokens, grouped from 683 with both at 16
    assert fill.select_arm(682, 6, 256, 16) == "gemv"
    assert fill.select_arm(683, 6, 256, 16) == "grouped"
    assert fill.select_arm(8, 6, 256, 1) == "gemv"        # decode floor
    assert fill.select_arm(9, 6, 256, 1) == "grouped"
    assert fill.select_arm(1000, 6, 256, 64) == "dequant"  # 16 <= 23.4 < 64
