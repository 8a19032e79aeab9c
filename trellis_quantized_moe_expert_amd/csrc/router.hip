// Router GEMM: one logit per (token, expert) from bf16 hidden states and a bf16 router
// weight, on the matrix cores with fp32 accumulation.
//
// The router GEMM that feeds top-k routing is named as a cost of its own on the
// 794-ms-decode-step page (PR #202, closing list of remaining un-owned items, item (3)):
// there it ran in FP32 on scalar cores behind a cast of the activations; here it reads the
// bf16 activations the experts read and runs v_mfma_f32_16x16x32_bf16.
//
// A workgroup owns one 32-expert x 32-token output tile and one of S chunks of the inputs;
// its W waves split the chunk again and add their partial tiles through LDS in ascending
// wave order.  The S chunk sums go to part[s][t][e]; the consumer (the top-k kernel, or the
// reduction kernel below when the caller wants the logits themselves) adds them in
// ascending s, so both see bit-identical logits.  With S = 1 the chunk sum is the logit.

#include "qtip_internal.h"

namespace qtip {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTE = 2;  // 16-expert blocks per wave (MFMA M)
constexpr int kTM = 2;  // 16-token blocks per wave (MFMA N)

// Fragments of one 128-input block for `rows` row blocks: lane (j, g) reads the 64
// contiguous bytes of inputs 32g..32g+31 of its row; MFMA step st takes 8 of them (K slots
// 8g..8g+7 <-> inputs 32g + 8st + 0..7).  Both operands use the same permutation of the
// contraction index, so the dot products are unchanged.
template <int R>
__device__ inline void load_block(u32x4 (&f)[R][4], const uint16_t* __restrict__ base, const uint32_t (&off)[R],
                                  int kb) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
      f[r][st] = *reinterpret_cast<const u32x4*>(base + (off[r] + (uint32_t)(kb * kKBlock + st * 8)));
  }
}

__global__ __launch_bounds__(kRouterMaxWaves * 64) void router_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int32_t n, int32_t E, int32_t H, int32_t S,
    int32_t tiles_e, int32_t groups, int32_t n_xcd, float* __restrict__ part) {
  __shared__ f32x4 red[kRouterMaxWaves][kTE * kTM][64];
  // Workgroup b runs on XCD b mod n_xcd; each XCD takes a contiguous range of (tile, chunk)
  // groups, i.e. a few token tiles with all their expert tiles, so each token's hidden state
  // is fetched into one XCD's L2 only.  Workgroups past the last group leave at once.
  const int per_xcd = (groups + n_xcd - 1) / n_xcd;
  const int grp = (int)(blockIdx.x % n_xcd) * per_xcd + (int)(blockIdx.x / n_xcd);
  if (grp >= groups) return;  // uniform over the workgroup, before any barrier
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int s = grp % S;
  const int tile = grp / S;
  const int e0 = (tile % tiles_e) * 16 * kTE;
  const int t0 = (tile / tiles_e) * 16 * kTM;
  const int j = lane & 15, g = lane >> 4;
  const int bpw = H / kKBlock / (S * W);       // 128-input blocks per wave
  const uint32_t k0 = (uint32_t)((s * W + wv) * bpw * kKBlock + 32 * g);

  // rows past E or n read the last valid row; their results are never stored
  uint32_t aoff[kTE], boff[kTM];
#pragma unroll
  for (int te = 0; te < kTE; ++te) {
    const int e = min(e0 + 16 * te + j, E - 1);
    aoff[te] = (uint32_t)e * (uint32_t)H + k0;
  }
#pragma unroll
  for (int tm = 0; tm < kTM; ++tm) {
    const int t = min(t0 + 16 * tm + j, n - 1);
    boff[tm] = (uint32_t)t * (uint32_t)H + k0;
  }

  f32x4 acc[kTE][kTM];
#pragma unroll
  for (int te = 0; te < kTE; ++te)
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm) acc[te][tm] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 an[kTE][4], bn[kTM][4];
  load_block<kTE>(an, w, aoff, 0);
  load_block<kTM>(bn, x, boff, 0);
  for (int kb = 0; kb < bpw; ++kb) {
    u32x4 a[kTE][4], b[kTM][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int te = 0; te < kTE; ++te) a[te][st] = an[te][st];
#pragma unroll
      for (int tm = 0; tm < kTM; ++tm) b[tm][st] = bn[tm][st];
    }
    if (kb + 1 < bpw) {  // the next block, in flight during this one's MFMAs
      load_block<kTE>(an, w, aoff, kb + 1);
      load_block<kTM>(bn, x, boff, kb + 1);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int te = 0; te < kTE; ++te) {
#pragma unroll
        for (int tm = 0; tm < kTM; ++tm)
          acc[te][tm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[te][st]),
                                                                __builtin_bit_cast(bf16x8, b[tm][st]), acc[te][tm],
                                                                0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int te = 0; te < kTE; ++te)
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm) red[wv][te * kTM + tm][lane] = acc[te][tm];
  __syncthreads();

  // Element q of the tile (q = ((te*kTM + tm)*64 + lane)*4 + r) is expert e0 + 16te + 4(lane/16) + r
  // of token t0 + 16tm + lane%16 (the MFMA D layout); the waves' values are added in order.
  const float* redf = reinterpret_cast<const float*>(&red[0][0][0]);
  constexpr int kTileElems = kTE * kTM * 64 * 4;
  float* out = part + (size_t)s * (size_t)n * (size_t)E;
  for (int q = threadIdx.x; q < kTileElems; q += blockDim.x) {
    float v = redf[q];
    for (int u = 1; u < W; ++u) v += redf[u * kTileElems + q];
    const int r = q & 3, ln = (q >> 2) & 63, blk = q >> 8;
    const int te = blk / kTM, tm = blk % kTM;
    const int e = e0 + 16 * te + 4 * (ln >> 4) + r;
    const int t = t0 + 16 * tm + (ln & 15);
    if (e < E && t < n) out[(size_t)t * E + e] = v;
  }
}

// logits[i] = sum over s ascending of part[s][i]: the same additions, in the same order,
// as the top-k kernel makes when it reads the partials itself.
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part, int32_t S, int64_t count,
                                                            float* __restrict__ logits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const float* col = part + i;
  float v = col[0];
  for (int s = 1; s < S; s += 8) {  // up to 8 loads in flight, then their additions in order
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = (s + k < S) ? col[(size_t)(s + k) * (size_t)count] : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s + k < S) v += t[k];
  }
  logits[i] = v;
}

}  // namespace

int32_t router_tiles(int32_t n, int32_t E) {
  return ((E + 16 * kTE - 1) / (16 * kTE)) * ((n + 16 * kTM - 1) / (16 * kTM));
}

// Input chunks per tile: enough workgroups to reach every CU (about 256), at most 4 partial
// sums for the consumer to add; a divisor of the H/128 input blocks.
int32_t router_split(int32_t n, int32_t E, int32_t H) {
  const int64_t tiles = router_tiles(n, E);
  const int32_t blocks = H / kKBlock;
  const int64_t want = (kRouterTargetGroups + tiles - 1) / tiles;
  int32_t best = 1;
  for (int32_t d = 1; d <= blocks && d <= kRouterMaxSplit && d <= want; ++d)
    if (blocks % d == 0) best = d;
  return best;
}

// Waves per workgroup: the largest divisor of the blocks of one chunk up to kRouterMaxWaves.
int32_t router_waves(int32_t H, int32_t S) {
  const int32_t per_chunk = H / kKBlock / S;
  int32_t best = 1;
  for (int32_t d = 1; d <= per_chunk && d <= kRouterMaxWaves; ++d)
    if (per_chunk % d == 0) best = d;
  return best;
}

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w, int32_t n, int32_t E, int32_t H, int32_t S,
                              int32_t n_xcd, float* part, hipStream_t stream) {
  const int32_t tiles_e = (E + 16 * kTE - 1) / (16 * kTE);
  const int32_t groups = router_tiles(n, E) * S;
  const int32_t W = router_waves(H, S);
  const int32_t xcd = n_xcd >= 1 ? n_xcd : 1;
  const int32_t grid = (groups + xcd - 1) / xcd * xcd;
  hipLaunchKernelGGL(router_gemm_kernel, dim3((unsigned)grid), dim3(W * 64), 0, stream, x, w, n, E, H, S, tiles_e,
                     groups, xcd, part);
  return hipGetLastError();
}

hipError_t launch_router_reduce(const float* part, int32_t S, int64_t count, float* logits, hipStream_t stream) {
  const int64_t grid = (count + 255) / 256;
  hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)grid), dim3(256), 0, stream, part, S, count, logits);
  return hipGetLastError();
}

}  // namespace qtip
