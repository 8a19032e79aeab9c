// Closed-form m-tile fill model and grouped-arm predicate (host only, header-only so the
// plan and the exported functions evaluate the same code).
//
// Source: m-tile occupancy page, PR #167 "gate the trellis grouped GEMM on m-tile
// occupancy, not token count".  Section "The cause is a threshold, not a kernel defect":
// under uniform routing n tokens wake E(1 - (1 - k/E)^n) of E experts on average, and
// the grouped arm's advantage is the mean number of pairs per woken expert against the
// m-tile height.  Section "The fix": select the grouped arm when that mean reaches the
// m-tile height; the decode-regime floor (n <= 8 always GEMV) stays; the predicate needs
// only host scalars, so it is safe during graph capture.
#pragma once

#include <cmath>
#include <cstdint>

namespace qtip {

// The pages' decode-regime floor (n <= 8 always takes the per-pair arm, a graph-capture safety
// rule there); a plan carries its own floor (qtip_moe_desc.decode_floor).
constexpr int32_t kDecodeRegimeMaxTokens = 8;
// Fused GEMV vs dequantize-materialise: the GEMV streams an expert's packed bytes once per
// pair; materialising writes the dense bf16 weights and reads them back, 2 x 16/2 = 16 times
// the 2-bit packed bytes.  The m-tile page's "Tests" section names the constant (16) and
// requires the grouped boundary not to leave a window for the dequantize arm between them.
constexpr int32_t kDequantTrafficRatio = 16;

inline double fill_woken_experts(int32_t n, int32_t k, int32_t E) {
  return (double)E * (1.0 - std::pow(1.0 - (double)k / (double)E, (double)n));
}

inline double fill_pairs_per_woken_expert(int32_t n, int32_t k, int32_t E) {
  return (double)n * (double)k / fill_woken_experts(n, k, E);
}

inline bool fill_args_ok(int32_t n, int32_t k, int32_t E, int32_t tile_m) {
  return n >= 1 && k >= 1 && E >= 1 && k <= E && tile_m >= 1;
}

inline bool fill_select_grouped(int32_t n, int32_t k, int32_t E, int32_t tile_m,
                                int32_t floor = kDecodeRegimeMaxTokens) {
  return n > floor && fill_pairs_per_woken_expert(n, k, E) >= (double)tile_m;
}

// Three-arm dispatch: 2 = grouped, 1 = fused GEMV, 3 = dequantize-materialise (the values of
// QTIP_ARM_GROUPED / _GEMV / _DEQUANT).
inline int32_t fill_select_arm(int32_t n, int32_t k, int32_t E, int32_t tile_m, int32_t dequant_ratio,
                               int32_t floor = kDecodeRegimeMaxTokens) {
  if (fill_select_grouped(n, k, E, tile_m, floor)) return 2;
  if (n <= floor || fill_pairs_per_woken_expert(n, k, E) < (double)dequant_ratio) return 1;
  return 3;
}

// Smallest n that selects the grouped arm.  Pairs per woken expert never decreases with n
// (n / (1 - q^n) has derivative proportional to 1 - x + x ln x >= 0 with x = q^n), so an
// upward scan finds the flip point; -1 if it lies beyond 2^30.
inline int32_t fill_min_tokens(int32_t k, int32_t E, int32_t tile_m, int32_t floor = kDecodeRegimeMaxTokens) {
  int32_t lo = 1, hi = 1;
  while (!fill_select_grouped(hi, k, E, tile_m, floor)) {
    lo = hi;
    if (hi >= (1 << 30)) return -1;
    hi *= 2;
  }
  while (lo < hi) {  // invariant: select(hi) true; select(n) false for every n < lo
    int32_t mid = lo + (hi - lo) / 2;
    if (fill_select_grouped(mid, k, E, tile_m, floor)) hi = mid; else lo = mid + 1;
  }
  return hi;
}

}  // namespace qtip
