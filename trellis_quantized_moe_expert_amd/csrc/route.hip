// Routing and binning kernels.
//
// Source: m-tile occupancy page, PR #167, section "The cause is a threshold, not a kernel
// defect": pairs are sorted by expert and the grouped kernel walks sum_e ceil(count_e /
// tile_m) m-tiles.  The arch-specialise page (PR #99, section "D18") requires the tile map
// to come from the same m-tile height the GEMM uses; here both read the plan's value.
//
// Readings fixed by the C ABI: top-k in descending logit order with ties to the lower
// expert index; router weights = softmax over the k selected logits; within an expert's
// bin pairs keep ascending pair id p = t*k + j (a stable counting sort), so the binning
// is unique and can be compared bit for bit.
#include "qtip_internal.h"

#include <cmath>

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

// One wave per token.  Each lane holds up to 16 logits (E <= 1024); k rounds of a wave-wide
// argmax under the order (value descending, index ascending) pick the experts in order: each
// lane's best, then the largest value over the wave and the lowest index holding it, both by
// DPP row scans and scalar reads (no LDS round trips).
__global__ __launch_bounds__(kRouteWaves * 64) void route_topk_kernel(const float* __restrict__ logits,
                                                                    int32_t n_part, int32_t n, int32_t E, int32_t k,
                                                                    int32_t* __restrict__ topk_idx,
                                                                    float* __restrict__ topk_w) {
  __shared__ float sel[kRouteWaves][kMaxTopK];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kRouteWaves + wv;
  if (t >= n) return;  // whole wave leaves together; no barrier follows
  const float* row = logits + (size_t)t * E;
  const size_t part_stride = (size_t)n * (size_t)E;
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = lane + 64 * q;
    v[q] = (e < E) ? row[e] : 0.0f;
  }
  // partial sums of the router GEMM's K chunks, added in ascending chunk order; the loads of
  // up to 4 chunks are issued before their additions so their latencies overlap
  if (n_part > 1) {
    for (int s = 1; s < n_part; s += 4) {
      float t[4][16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int e = lane + 64 * q;
          t[i][q] = (s + i < n_part && e < E) ? row[(size_t)(s + i) * part_stride + e] : 0.0f;
        }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (s + i < n_part) v[q] += t[i][q];
    }
  }
  uint32_t taken = 0;
  for (int jj = 0; jj < k; ++jj) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
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
    if (lane == 0) {
      topk_idx[(size_t)t * k + jj] = be;
      sel[wv][jj] = bv;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // softmax over the k selected logits, max subtracted first (sel[0] is the largest)
  float ex = 0.0f;
  if (lane < k) ex = expf(sel[wv][lane] - sel[wv][0]);
  float z = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  if (lane < k) topk_w[(size_t)t * k + lane] = ex / z;
}

// Inclusive scan over a wave: DPP row shifts scan each 16-lane row, then the last lane of row 0
// is added into rows 1 and 3 and the last lane of row 1 (now rows 0-1) into rows 2 and 3.
__device__ inline int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

struct Scan4 {
  int a, b, c, d;
};

// Inclusive scans of four values per thread across a 1024-thread workgroup, sharing one
// exchange of the wave totals.
__device__ inline Scan4 block_inclusive_scan4(Scan4 x, Scan4* wave_tot) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  x.a = wave_inclusive_scan(x.a);
  x.b = wave_inclusive_scan(x.b);
  x.c = wave_inclusive_scan(x.c);
  x.d = wave_inclusive_scan(x.d);
  if (lane == 63) wave_tot[wv] = x;
  __syncthreads();
  for (int w = 0; w < wv; ++w) {
    const Scan4 t = wave_tot[w];
    x.a += t.a;
    x.b += t.b;
    x.c += t.c;
    x.d += t.d;
  }
  __syncthreads();
  return x;
}

// Stable counting sort of the n*k pairs by expert, plus the m-tile map and the unit map
// (units = runs of up to unit_pairs pairs of one expert; each unit is one decode of the
// expert's weights in the expert kernels; unit_map/n_units may be NULL to skip them).
// One workgroup of 1024 threads.
__global__ __launch_bounds__(kBinThreads) void bin_kernel(const int32_t* __restrict__ topk_idx, int32_t P, int32_t E,
                                                          int32_t tile_m, int32_t unit_pairs,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pair,
                                                          int32_t* __restrict__ tile_map, int32_t* __restrict__ n_tiles,
                                                          int32_t* __restrict__ unit_map,
                                                          int32_t* __restrict__ n_units,
                                                          int32_t* __restrict__ padded_pair,
                                                          int32_t* __restrict__ unit_pad,
                                                          int32_t* __restrict__ n_pad) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int running[kMaxExperts];
  __shared__ int pad_shift[kMaxExperts];  // padded position - binned position, per expert
  __shared__ int wave_cnt[kExpertWaves][kMaxExperts];
  __shared__ Scan4 wave_tot[kExpertWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;

  for (int e = tid; e < E; e += kBinThreads) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kBinThreads) {
    const int e = topk_idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // exclusive scans of counts, tiles per expert and units per expert (E <= 1024 = threads)
  const int c = (tid < E) ? cnt[tid] : 0;
  const int nt = (c + tile_m - 1) / tile_m;
  const int nu = (c + unit_pairs - 1) / unit_pairs;
  const int pc = (c + 15) & ~15;  // the bin rounded up to whole 16-pair MFMA blocks
  const Scan4 sc = block_inclusive_scan4(Scan4{c, nt, nu, pc}, wave_tot);
  const int c_incl = sc.a, t_incl = sc.b, u_incl = sc.c, p_incl = sc.d;
  if (tid < E) {
    const int off = c_incl - c;
    const int poff = p_incl - pc;
    counts[tid] = c;
    offsets[tid] = off;
    running[tid] = off;
    pad_shift[tid] = poff - off;
    if (padded_pair)
      for (int q = c; q < pc; ++q) padded_pair[poff + q] = -1;
    for (int q = 0; unit_pad && q < nu; ++q) unit_pad[u_incl - nu + q] = poff + q * unit_pairs;
    int tb = t_incl - nt;
    for (int q = 0; q < nt; ++q) {
      tile_map[3 * (tb + q) + 0] = tid;
      tile_map[3 * (tb + q) + 1] = off + q * tile_m;
      tile_map[3 * (tb + q) + 2] = min(tile_m, c - q * tile_m);
    }
    int ub = u_incl - nu;
    for (int q = 0; unit_map && q < nu; ++q) {
      unit_map[3 * (ub + q) + 0] = tid;
      unit_map[3 * (ub + q) + 1] = off + q * unit_pairs;
      unit_map[3 * (ub + q) + 2] = min(unit_pairs, c - q * unit_pairs);
    }
  }
  if (tid == E - 1) {
    offsets[E] = c_incl;
    *n_tiles = t_incl;
    if (n_units) *n_units = u_incl;
    if (n_pad) *n_pad = p_incl;
  }
  __syncthreads();

  // stable scatter, 1024 pairs per round: rank inside the wave from a bitwise match of
  // the expert id, then the counts of earlier waves and earlier rounds
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < P; base += kBinThreads) {
    for (int i = tid; i < kExpertWaves * E; i += kBinThreads) (&wave_cnt[0][0])[(i / E) * kMaxExperts + (i % E)] = 0;
    const int p = base + tid;
    const int ep = (p < P) ? topk_idx[p] : E;
    const bool valid = ep >= 0 && ep < E;
    const int e = valid ? ep : E;  // E: one bucket for idle lanes and out-of-range ids
    uint64_t peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    __syncthreads();
    if (valid && rank == 0) wave_cnt[wv][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = running[e] + rank;
      for (int w = 0; w < wv; ++w) pos += wave_cnt[w][e];
      sorted_pair[pos] = p;
      if (padded_pair) padded_pair[pos + pad_shift[e]] = p;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kBinThreads) {
      int add = 0;
      for (int w = 0; w < kExpertWaves; ++w) add += wave_cnt[w][ee];
      running[ee] += add;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int32_t n_part, int32_t n, int32_t E, int32_t k,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  const int grid = (n + kRouteWaves - 1) / kRouteWaves;
  hipLaunchKernelGGL(route_topk_kernel, dim3(grid), dim3(kRouteWaves * 64), 0, stream, logits, n_part, n, E, k,
                     topk_idx, topk_w);
  return hipGetLastError();
}

hipError_t launch_bin(const int32_t* topk_idx, int32_t n_pairs, int32_t E, int32_t tile_m, int32_t unit_pairs,
                      int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* tile_map, int32_t* n_tiles,
                      int32_t* unit_map, int32_t* n_units, int32_t* padded_pair, int32_t* unit_pad, int32_t* n_pad,
                      hipStream_t stream) {
  hipLaunchKernelGGL(bin_kernel, dim3(1), dim3(kBinThreads), 0, stream, topk_idx, n_pairs, E, tile_m, unit_pairs,
                     counts, offsets, sorted_pair, tile_map, n_tiles, unit_map, n_units, padded_pair, unit_pad,
                     n_pad);
  return hipGetLastError();
}

}  // namespace qtip
