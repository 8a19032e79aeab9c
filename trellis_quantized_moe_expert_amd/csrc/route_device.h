// Routing of one token by one wave: shared by the routing kernels and by the expert pass that
// routes a small batch itself.  Not part of the ABI.
//
// Source: m-tile occupancy page, PR #167, "The cause is a threshold, not a kernel defect" (pairs
// are routed to their top-k experts, then binned by expert).  Readings fixed by the C ABI: top-k
// in descending logit order with ties to the lower expert index; router weights = softmax over
// the k selected logits.
#pragma once

#include <cmath>

#include "qtip_internal.h"

namespace qtip {

namespace {

__device__ inline bool beats(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

// Order-preserving integer key of a float under `>` (+0 and -0 map to the same key, as they
// compare equal; NaN, never selected by `beats`, maps below every number).
__device__ inline uint32_t order_key(float v) {
  if (v != v) return 0u;
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide max / min of one 32-bit value per lane without the LDS: an inclusive scan inside
// each 16-lane row by DPP row shifts (lanes past the row start keep their own value), then the
// four row results (lanes 15, 31, 47, 63) combined in scalar registers.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 15), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 47), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(a, b), max(c, d));
}

__device__ inline int wave_min_i32(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x111, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x112, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x114, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xF, 0xF, false));
  const int a = __builtin_amdgcn_readlane(v, 15), b = __builtin_amdgcn_readlane(v, 31);
  const int c = __builtin_amdgcn_readlane(v, 47), d = __builtin_amdgcn_readlane(v, 63);
  return min(min(a, b), min(c, d));
}

// Top-k and softmax of token t by one wave.  Each lane holds Q logits (E <= 64 Q); k rounds
// of a wave-wide argmax under the order (value descending, index ascending) pick the experts
// in order: each lane's best, then the largest value over the wave and the lowest index
// holding it, both by DPP row scans and scalar reads (no LDS round trips).
//
// The expert ids go to idx (and to idx2 unless it is NULL: a second copy, e.g. workgroup
// memory and global memory), the router weights to topk_w unless it is NULL.
template <int Q>
__device__ __attribute__((always_inline)) inline void route_token(const float* __restrict__ logits, int32_t n_part,
                                                                  int32_t n, int32_t E, int32_t k, int t,
                                                                  int32_t* idx, int32_t* idx2, float* topk_w) {
  const int lane = threadIdx.x & 63;
  float sel = 0.0f;  // lane j: the j-th selected logit
  const float* row = logits + (size_t)t * E;
  const size_t part_stride = (size_t)n * (size_t)E;
  float v[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    v[q] = (e < E) ? row[e] : 0.0f;
  }
  // partial sums of the router GEMM's K chunks, added in ascending chunk order; the loads of
  // up to 4 chunks are issued before their additions so their latencies overlap
  for (int s = 1; s < n_part; s += 4) {
    float t4[4][Q];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        t4[c][q] = (s + c < n_part && e < E) ? row[(size_t)(s + c) * part_stride + e] : 0.0f;
      }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (s + c < n_part) v[q] += t4[c][q];
  }
  uint32_t taken = 0;
  for (int jj = 0; jj < k; ++jj) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + 64 * q;
      if (e < E && !((taken >> q) & 1u) && beats(v[q], e, bv, be)) {
        bv = v[q];
        be = e;
      }
    }
    // the wave's winner under the same order: the largest value, then the lowest index
    // among the lanes holding it (lanes without a candidate hold index INT_MAX)
    const uint32_t kmax = wave_max_u32(be < E ? order_key(bv) : 0u);
    const int cand = (be < E && order_key(bv) == kmax) ? be : 0x7fffffff;
    const int win = wave_min_i32(cand);
    // the winning lane's own best is the winner: take its value (the sign of a zero included)
    if (win < E) bv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), win & 63));
    be = win;
    // non-finite logits can leave no winner (be stays out of range); the pair is then
    // recorded with an out-of-range expert id, which binning ignores
    if (be < E && (be & 63) == lane) taken |= 1u << (be >> 6);
    const float b0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
    if (lane == jj) sel = b0;
    if (lane == 0) {
      idx[(size_t)t * k + jj] = be;
      if (idx2) idx2[(size_t)t * k + jj] = be;
    }
  }
  // softmax over the k selected logits, max subtracted first (lane 0's is the largest)
  const float sel0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sel), 0));
  float ex = 0.0f;
  if (lane < k) ex = expf(sel - sel0);
  float z = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  if (topk_w && lane < k) topk_w[(size_t)t * k + lane] = ex / z;
}

}  // namespace

}  // namespace qtip
