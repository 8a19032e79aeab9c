"""Closed-form m-tile fill model and dispatch predicate, oracle side (test infrastructure only).

Source: the gate-the-grouped-GEMM page (PR #167 "gate the trellis grouped GEMM on
m-tile occupancy, not token count"):
* section "The cause is a threshold, not a kernel defect": under uniform routing of
  n tokens to k of E experts, the expected number of distinct (woken) experts is
  E*(1 - (1 - k/E)**n); pairs per woken expert is n*k divided by that; fill is that
  ratio over the m-tile height.
* section "The fix": the grouped arm is selected when pairs per woken expert reach
  the m-tile height (an average m-tile is full); the decode-regime floor (n <= 8
  always takes the per-pair arm) is kept, and an explicit pin overrides both
  (post-merge note).
* section "Tests": the boundary is the smallest n for which the predicate holds; the
  grouped boundary and the fused-GEMV boundary are set by two separate constants (both
  16 there) and must leave no token range that falls through to the third arm, which
  dequantizes the experts into dense weights and multiplies those.

Reading for the third arm (the pages name the constant, not its formula): the fused
GEMV streams each woken expert's packed bytes once per pair, while materialising
writes the dense bf16 weights and reads them back, 2 x 16/2 = 16 times the packed
2-bit bytes; so the fused GEMV is kept while pairs per woken expert < 16 (the
traffic ratio), the grouped arm takes over at its own threshold, and anything in
between goes to the dequantize arm.

The expected tile count is the binomial expectation of sum_e ceil(count_e / tile_m)
with count_e ~ Binomial(n, k/E) (each token picks k distinct experts uniformly).
"""
from __future__ import annotations

import math

DECODE_REGIME_MAX_TOKENS = 8
DEQUANT_TRAFFIC_RATIO = 16


def woken_experts(n: int, k: int, E: int) -> float:
    return E * (1.0 - (1.0 - k / E) ** n)


def pairs_per_woken_expert(n: int, k: int, E: int) -> float:
    return n * k / woken_experts(n, k, E)


def tile_fill(n: int, k: int, E: int, tile_m: int) -> float:
    return pairs_per_woken_expert(n, k, E) / tile_m


def tiles_amortize(n: int, k: int, E: int, tile_m: int) -> bool:
    return pairs_per_woken_expert(n, k, E) >= tile_m


def select_grouped(n: int, k: int, E: int, tile_m: int,
                   floor: int = DECODE_REGIME_MAX_TOKENS) -> bool:
    return n > floor and tiles_amortize(n, k, E, tile_m)


def select_arm(n: int, k: int, E: int, grouped_threshold: int, dequant_ratio: int = DEQUANT_TRAFFIC_RATIO,
               floor: int = DECODE_REGIME_MAX_TOKENS) -> str:
    """'grouped', 'gemv' or 'dequant' for n tokens (the three-arm dispatch)."""
    if select_grouped(n, k, E, grouped_threshold, floor):
        return "grouped"
    if n <= floor or pairs_per_woken_expert(n, k, E) < dequant_ratio:
        return "gemv"
    return "dequant"


def dequant_tokens(k: int, E: int, grouped_threshold: int, dequant_ratio: int, n_max: int,
                   floor: int = DECODE_REGIME_MAX_TOKENS) -> list:
    """Every n in [1, n_max] that the three-arm dispatch sends to the dequantize arm."""
    return [n for n in range(1, n_max + 1)
            if select_arm(n, k, E, grouped_threshold, dequant_ratio, floor) == "dequant"]


def min_tokens_grouped(k: int, E: int, tile_m: int, floor: int = DECODE_REGIME_MAX_TOKENS) -> int:
    """Smallest n for which select_grouped holds, by a plain upward scan."""
    n = 1
    while not select_grouped(n, k, E, tile_m, floor):
        n += 1
    return n


def expected_tiles(n: int, k: int, E: int, tile_m: int) -> float:
    """E * sum_c P[Binomial(n, k/E) = c] * ceil(c / tile_m)."""
    p = k / E
    total = 0.0
    for c in range(1, n + 1):
        logpmf = (math.lgamma(n + 1) - math.lgamma(c + 1) - math.lgamma(n - c + 1)
                  + c * math.log(p) + ((n - c) * math.log1p(-p) if p < 1 else (0.0 if c == n else -math.inf)))
        total += math.exp(logpmf) * math.ceil(c / tile_m)
    return E * total
