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
#include "route_device.h"

#include <cmath>

namespace qtip {

namespace {

// One wave per token.
template <int Q>
__global__ __launch_bounds__(kRouteWaves * 64) void route_topk_kernel(const float* __restrict__ logits,
                                                                    int32_t n_part, int32_t n, int32_t E, int32_t k,
                                                                    int32_t* __restrict__ topk_idx,
                                                                    float* __restrict__ topk_w) {
  const int t = blockIdx.x * kRouteWaves + (int)(threadIdx.x >> 6);
  if (t >= n) return;  // whole wave leaves together; no barrier follows
  route_token<Q>(logits, n_part, n, E, k, t, topk_idx, nullptr, topk_w);
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

// Values scanned together across the binning workgroup: a pair count, m-tiles, units and
// padded pairs per expert, and the expert's decodes in the two expert passes.
struct Scan6 {
  int v[6];
};

// Inclusive scans of six values per thread across a 1024-thread workgroup, sharing one
// exchange of the wave totals (left in wave_tot: their sum is the workgroup total).
__device__ inline Scan6 block_inclusive_scan6(Scan6 x, Scan6* wave_tot) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 6; ++i) x.v[i] = wave_inclusive_scan(x.v[i]);
  if (lane == 63) wave_tot[wv] = x;
  __syncthreads();
  for (int w = 0; w < wv; ++w) {
    const Scan6 t = wave_tot[w];
#pragma unroll
    for (int i = 0; i < 6; ++i) x.v[i] += t.v[i];
  }
  __syncthreads();
  return x;
}

// The decode units of one expert pass: runs of up to unit_pairs pairs of one expert, each one
// decode of the expert's rows in that pass (unit_pairs = the pass kernel's pairs per decode).
// map: (expert, first binned position, pairs) per unit; pad: each unit's first padded position
// (NULL without the padded space); count: the number of units.  map NULL: no units.
struct UnitOut {
  int32_t unit_pairs;
  int32_t* map;
  int32_t* pad;
  int32_t* count;
};

// A lane's expert id ep (E for none), its rank among the wave's lanes holding the same valid
// expert (a bitwise match of the id over nbits ballots) and that group's size.
__device__ inline void peer_rank(int ep, int E, int nbits, uint64_t lt_mask, int& e, int& rank, int& group) {
  e = (ep >= 0 && ep < E) ? ep : E;  // E: one bucket for idle lanes and out-of-range ids
  uint64_t peers = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const uint64_t m = __ballot((e >> b) & 1);
    peers &= ((e >> b) & 1) ? m : ~m;
  }
  rank = __popcll(peers & lt_mask);
  group = __popcll(peers);
}

// Stable counting sort of the n*k pairs by expert, plus the m-tile map and the decode units of
// the two expert passes (ug: the fused gate/up pass, ud: the down pass).  Run by one workgroup
// of 1024 threads.
__device__ __attribute__((always_inline)) inline void bin_pairs(const int32_t* __restrict__ topk_idx, int32_t P, int32_t E, int32_t tile_m,
                                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                 int32_t* __restrict__ sorted_pair, int32_t* __restrict__ tile_map,
                                 int32_t* __restrict__ n_tiles, int32_t* __restrict__ padded_pair,
                                 int32_t* __restrict__ n_pad, const UnitOut& ug, const UnitOut& ud) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int pad_shift[kMaxExperts];  // padded position - binned position, per expert
  __shared__ int wave_cnt[kExpertWaves][kMaxExperts];  // per wave: its pairs of each expert, then their first slot
  __shared__ Scan6 wave_tot[kExpertWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;

  // Wave w owns pairs [w C, (w + 1) C), C a multiple of 64, and walks them 64 at a time in
  // ascending order, twice: first counting its pairs of each expert, then, once every wave's
  // counts are turned into its first slot in each expert's bin, placing them.  A pair's rank
  // among the lanes of its 64 holding the same expert comes from a bitwise match of the expert
  // id over ballots; the lowest such lane advances the wave's count.  Bins keep ascending pair
  // order (waves own ascending chunks), and no barrier falls inside the walks.
  const int C = ((P + kExpertWaves - 1) / kExpertWaves + 63) & ~63;
  const int p_lo = wv * C, p_hi = min(P, p_lo + C);
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the first kBinCached groups of 64 of the wave's expert ids are loaded at once and kept for
  // both walks (one memory round trip instead of one per group); later groups load as needed
  int cached[kBinCached];
#pragma unroll
  for (int i = 0; i < kBinCached; ++i) {
    const int p = p_lo + 64 * i + lane;
    cached[i] = (p < p_hi) ? topk_idx[p] : E;
  }
  for (int e = lane; e < E; e += 64) wave_cnt[wv][e] = 0;
  auto count = [&](int ep) {
    int e, rank, group;
    peer_rank(ep, E, nbits, lt_mask, e, rank, group);
    if (e < E && rank == 0) wave_cnt[wv][e] += group;
  };
#pragma unroll
  for (int i = 0; i < kBinCached; ++i)
    if (p_lo + 64 * i < p_hi) count(cached[i]);
  for (int i = kBinCached; p_lo + 64 * i < p_hi; ++i) {
    const int p = p_lo + 64 * i + lane;
    count(p < p_hi ? topk_idx[p] : E);
  }
  __syncthreads();
  if (tid < E) {
    int c = 0;
    for (int w = 0; w < kExpertWaves; ++w) c += wave_cnt[w][tid];
    cnt[tid] = c;
  }

  // exclusive scans of counts, m-tiles, padded pairs and both passes' units per expert
  // (E <= 1024 = threads)
  const int c = (tid < E) ? cnt[tid] : 0;  // written by this thread
  const int nt = (c + tile_m - 1) / tile_m;
  const int pc = (c + 15) & ~15;  // the bin rounded up to whole 16-pair MFMA blocks
  const int nug = ug.map ? (c + ug.unit_pairs - 1) / ug.unit_pairs : 0;
  const int nud = ud.map ? (c + ud.unit_pairs - 1) / ud.unit_pairs : 0;
  const Scan6 sc = block_inclusive_scan6(Scan6{{c, nt, pc, nug, nud, 0}}, wave_tot);
  const int c_incl = sc.v[0], t_incl = sc.v[1], p_incl = sc.v[2];
  if (tid < E) {
    const int off = c_incl - c;
    const int poff = p_incl - pc;
    counts[tid] = c;
    offsets[tid] = off;
    int run = off;  // each wave's first slot in the bin: the pairs of earlier waves come first
    for (int w = 0; w < kExpertWaves; ++w) {
      const int nw = wave_cnt[w][tid];
      wave_cnt[w][tid] = run;
      run += nw;
    }
    pad_shift[tid] = poff - off;
    if (padded_pair)
      for (int q = c; q < pc; ++q) padded_pair[poff + q] = -1;
    int tb = t_incl - nt;
    for (int q = 0; q < nt; ++q) {
      tile_map[3 * (tb + q) + 0] = tid;
      tile_map[3 * (tb + q) + 1] = off + q * tile_m;
      tile_map[3 * (tb + q) + 2] = min(tile_m, c - q * tile_m);
    }
    auto units = [&](const UnitOut& uo, int nu, int u_incl) {
      const int ub = u_incl - nu;
      for (int q = 0; q < nu; ++q) {
        uo.map[3 * (ub + q) + 0] = tid;
        uo.map[3 * (ub + q) + 1] = off + q * uo.unit_pairs;
        uo.map[3 * (ub + q) + 2] = min(uo.unit_pairs, c - q * uo.unit_pairs);
        if (uo.pad) uo.pad[ub + q] = poff + q * uo.unit_pairs;
      }
    };
    if (ug.map) units(ug, nug, sc.v[3]);
    if (ud.map) units(ud, nud, sc.v[4]);
  }
  if (tid == E - 1) {
    offsets[E] = c_incl;
    *n_tiles = t_incl;
    if (ug.map) *ug.count = sc.v[3];
    if (ud.map) *ud.count = sc.v[4];
    if (n_pad) *n_pad = p_incl;
  }
  __syncthreads();

  auto place = [&](int ep, int p) {
    int e, rank, group;
    peer_rank(ep, E, nbits, lt_mask, e, rank, group);
    if (e < E) {
      const int pos = wave_cnt[wv][e] + rank;  // every lane reads before the lowest lane advances it
      sorted_pair[pos] = p;
      if (padded_pair) padded_pair[pos + pad_shift[e]] = p;
      if (rank == 0) wave_cnt[wv][e] = pos + group;
    }
  };
#pragma unroll
  for (int i = 0; i < kBinCached; ++i)
    if (p_lo + 64 * i < p_hi) place(cached[i], p_lo + 64 * i + lane);
  for (int i = kBinCached; p_lo + 64 * i < p_hi; ++i) {
    const int p = p_lo + 64 * i + lane;
    place(p < p_hi ? topk_idx[p] : E, p);
  }
}

__global__ __launch_bounds__(kBinThreads) void bin_kernel(const int32_t* __restrict__ topk_idx, int32_t P, int32_t E,
                                                          int32_t tile_m, int32_t* counts, int32_t* offsets,
                                                          int32_t* sorted_pair, int32_t* tile_map, int32_t* n_tiles,
                                                          int32_t* padded_pair, int32_t* n_pad, UnitOut ug, UnitOut ud) {
  bin_pairs(topk_idx, P, E, tile_m, counts, offsets, sorted_pair, tile_map, n_tiles, padded_pair, n_pad, ug, ud);
}

// Routing and binning of a small batch (n <= kFusedRouteMaxTokens) in one workgroup: its waves
// take a token each, then, once every pair is routed (the barrier makes the workgroup's stores
// of topk_idx visible to all of it), the same workgroup bins them.  Saves a launch and its
// latency where both steps are latency-bound.
template <int Q>
__global__ __launch_bounds__(kBinThreads) void route_bin_kernel(const float* __restrict__ logits, int32_t n_part,
                                                                int32_t n, int32_t E, int32_t k, int32_t* topk_idx,
                                                                float* topk_w, int32_t tile_m, int32_t* counts,
                                                                int32_t* offsets, int32_t* sorted_pair,
                                                                int32_t* tile_map, int32_t* n_tiles,
                                                                int32_t* padded_pair, int32_t* n_pad, UnitOut ug,
                                                                UnitOut ud) {
  const int t = (int)(threadIdx.x >> 6);
  if (t < n) route_token<Q>(logits, n_part, n, E, k, t, topk_idx, nullptr, topk_w);
  __syncthreads();
  bin_pairs(topk_idx, n * k, E, tile_m, counts, offsets, sorted_pair, tile_map, n_tiles, padded_pair, n_pad, ug, ud);
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int32_t n_part, int32_t n, int32_t E, int32_t k,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  const int grid = (n + kRouteWaves - 1) / kRouteWaves;
  if (E <= 256)
    hipLaunchKernelGGL(route_topk_kernel<4>, dim3(grid), dim3(kRouteWaves * 64), 0, stream, logits, n_part, n, E, k,
                       topk_idx, topk_w);
  else if (E <= 512)
    hipLaunchKernelGGL(route_topk_kernel<8>, dim3(grid), dim3(kRouteWaves * 64), 0, stream, logits, n_part, n, E, k,
                       topk_idx, topk_w);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, dim3(grid), dim3(kRouteWaves * 64), 0, stream, logits, n_part, n, E, k,
                       topk_idx, topk_w);
  return hipGetLastError();
}

namespace {

UnitOut unit_out(const UnitMaps* um, int pass) {
  if (!um) return UnitOut{1, nullptr, nullptr, nullptr};
  return UnitOut{um->unit_pairs[pass], um->map[pass], um->pad[pass], um->count[pass]};
}

bool units_ok(const UnitMaps* um) {
  if (!um) return true;
  for (int i = 0; i < 2; ++i)
    if (!um->map[i] || !um->count[i] || um->unit_pairs[i] < 1 || um->unit_pairs[i] > kUnitMaxPairs) return false;
  return true;
}

}  // namespace

hipError_t launch_bin(const int32_t* topk_idx, int32_t n_pairs, int32_t E, int32_t tile_m, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_pair, int32_t* tile_map, int32_t* n_tiles,
                      int32_t* padded_pair, int32_t* n_pad, const UnitMaps* units, hipStream_t stream) {
  if (!units_ok(units)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bin_kernel, dim3(1), dim3(kBinThreads), 0, stream, topk_idx, n_pairs, E, tile_m, counts, offsets,
                     sorted_pair, tile_map, n_tiles, padded_pair, n_pad, unit_out(units, 0), unit_out(units, 1));
  return hipGetLastError();
}

hipError_t launch_route_bin(const float* logits, int32_t n_part, int32_t n, int32_t E, int32_t k, int32_t* topk_idx,
                            float* topk_w, int32_t tile_m, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                            int32_t* tile_map, int32_t* n_tiles, int32_t* padded_pair, int32_t* n_pad,
                            const UnitMaps* units, hipStream_t stream) {
  if (n < 1 || n > kFusedRouteMaxTokens || !units_ok(units)) return hipErrorInvalidValue;
  auto kernel = E <= 256 ? route_bin_kernel<4> : E <= 512 ? route_bin_kernel<8> : route_bin_kernel<16>;
  hipLaunchKernelGGL(kernel, dim3(1), dim3(kBinThreads), 0, stream, logits, n_part, n, E, k, topk_idx, topk_w, tile_m,
                     counts, offsets, sorted_pair, tile_map, n_tiles, padded_pair, n_pad, unit_out(units, 0),
                     unit_out(units, 1));
  return hipGetLastError();
}

}  // namespace qtip
