// Expert matmul kernels: trellis decode fused into the multiply, plus the combine.
//
// Sources:
//  - arch-specialise page, PR #99, section "The two levers": the grouped kernel stages
//    packed 2-bit bytes, decodes them on chip and multiplies; full-size weights never
//    materialise.  Lever 2 (contiguous-run decode): each thread owns a run of 32
//    consecutive symbols of one weight row, seeds the state once from its window and then
//    steps the recurrence.  Lever 1: decode work is (number of m-tiles) x (weights per
//    expert), so fewer, fuller tiles per expert means less decode and less traffic.
//  - m-tile occupancy page, PR #167, "The cause is a threshold": the grouped kernel walks
//    the expert-binned m-tiles; the per-pair GEMV is the arm for low fill.
//
// gfx950 design (what differs from the pages' CUDA kernels):
//  - The 65536-entry LUT, narrowed to bf16, lives in LDS (128 KiB of the 160 KiB); one
//    workgroup of 8, 12 or 16 waves per CU, persistent over wave-sized tasks.  Random 2-byte LUT
//    gathers are the decode's bottleneck, so decoded weights go straight into MFMA B-operand
//    registers instead of through an LDS weight tile, and activations are read from global
//    memory (L2-resident) into A-operand registers.  (Small GEMV launches also keep partial
//    sums in the rest of LDS; see gemv_split_tasks.)
//  - A wave task is one decode unit (the binned pairs of one expert that one decode serves:
//    up to 16, 32, 48 or 64 on the grouped arm, 1 to 4 on the GEMV arm) x 16 NT output rows x all
//    inputs.  Lane (j = lane%16, g = lane/16) decodes row j of each 16-row block; within each
//    128-input block lane group g owns the contiguous 32-symbol run [32g, 32g+32), loaded as
//    8 bytes plus one look-ahead dword (the next 7 symbols, wrapping to the row start at the
//    row end: the window is circular).  The contraction index is permuted accordingly: MFMA
//    step s of a block pairs K slot 8g+t with input 32g + 8s + t, for both operands, which
//    leaves the dot products unchanged.
//  - Grouped arm: v_mfma_f32_16x16x32_bf16 per 16-pair row block.  GEMV arm: the same
//    decoded registers feed VALU bf16 dot products per pair.
#include "expert_body.h"

namespace qtip {

namespace {

// Activations of the grouped arm in fragment order: one thread per 16-byte fragment slot
// (padded 16-row block, 128-input block kb, MFMA step st, lane j + 16g) copies inputs
// kb*128 + 32g + 8st .. +7 of its padded position's token row, so consecutive threads write
// consecutive 16-byte slots.  Padding slots are left as they are: only the MFMA rows of padded
// positions read them, and those rows' results are never stored (each output row of an MFMA
// depends on its own A row only).
__global__ __launch_bounds__(256) void pack_act_kernel(const uint16_t* __restrict__ x,
                                                       const int32_t* __restrict__ padded_pair,
                                                       const int32_t* __restrict__ n_pad, int32_t k, int32_t H,
                                                       int32_t n_pad_max, uint16_t* __restrict__ xs) {
  // one thread per (padded 16-row block, 128-input block, lane): it reads the 64 contiguous
  // bytes of its four MFMA steps and writes them to the four step slots, 1 KiB apart
  const int kblocks = H / kKBlock;
  const int npad = min(*n_pad, n_pad_max);
  const long items = (long)(npad >> 4) * kblocks * 64;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < items; i += (long)gridDim.x * 256) {
    const int lane = (int)(i & 63);
    const long rest = i >> 6;
    const int kb = (int)(rest % kblocks);
    const int rb = (int)(rest / kblocks);
    const int pair = padded_pair[rb * 16 + (lane & 15)];
    if (pair < 0) continue;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)(pair / k) * H + kb * kKBlock + 32 * (lane >> 4));
    u32x4 v[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) v[st] = src[st];
#pragma unroll
    for (int st = 0; st < 4; ++st)
      *reinterpret_cast<u32x4*>(xs + dense_fragment_offset(rb, kb, st, lane, kblocks)) = v[st];
  }
}

// out[t] = sum_j w[t,j] * y[t*k+j], j ascending, fp32; one thread per 4 outputs.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      int32_t n, int32_t k, int32_t H, void* __restrict__ out,
                                                      int out_bf16) {
  const int h4 = H >> 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)n * h4) return;
  const int t = (int)(idx / h4), c = (int)(idx - (long)t * h4) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // up to 8 rows' loads are issued before their (j-ascending) multiply-adds
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 v[8];
    float wt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (j0 + i < k) {
        wt[i] = w[(size_t)t * k + j0 + i];
        v[i] = *reinterpret_cast<const float4*>(y + ((size_t)t * k + j0 + i) * H + c);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (j0 + i < k) {
        acc.x = fmaf(wt[i], v[i].x, acc.x);
        acc.y = fmaf(wt[i], v[i].y, acc.y);
        acc.z = fmaf(wt[i], v[i].z, acc.z);
        acc.w = fmaf(wt[i], v[i].w, acc.w);
      }
  }
  if (out_bf16) {
    uint2 o;
    o.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
    o.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * H + c) = o;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (size_t)t * H + c) = acc;
  }
}

__global__ void witness_kernel(int32_t* out) { out[0] = kWitnessValue; }

// The decode's bottleneck in isolation: random 2-byte gathers from a 128 KiB LDS table.  Each
// lane draws 16 even byte offsets below 2^17 (xorshift32) and, per round, gathers them all after
// XOR-ing with a round-dependent even mask below 2^17, so every address stays inside the table.
__global__ __launch_bounds__(1024, 1) void gather_probe_kernel(int32_t rounds, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint16_t table[kLutEntries];
  for (int i = threadIdx.x; i < kLutEntries; i += blockDim.x) table[i] = (uint16_t)(i * 40503u);
  __syncthreads();
  uint32_t st = 0x9E3779B9u ^ ((blockIdx.x * 1024u + threadIdx.x) * 2654435761u);
  uint32_t a[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    st ^= st << 13;
    st ^= st >> 17;
    st ^= st << 5;
    a[q] = (st & 0xFFFFu) << 1;
  }
  uint32_t acc = 0;
  const char* base = reinterpret_cast<const char*>(table);
  for (int it = 0; it < rounds; ++it) {
    const uint32_t m = ((uint32_t)it * 0x9E3779B9u) & 0x1FFFEu;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc += *reinterpret_cast<const uint16_t*>(base + (a[q] ^ m));
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

template <class CFG>
struct CfgInfo {
  static void get(int arm, VariantInfo& v) {
    if (arm == kArmDense) {
      v.waves = CfgDense::kWaves;
      v.rows_per_task = CfgDense::kRows;
      v.pairs_per_decode = CfgDense::kNSub * 16;
      v.input_split = false;
      return;
    }
    v.waves = CFG::kWaves;
    v.rows_per_task = CFG::kRows;
    v.pairs_per_decode = arm == kArmGrouped ? CFG::kNSub * 16 : CFG::kGPairs;
    v.input_split = arm == kArmGemv && GemvSplit<CFG>::kFits;
  }
};

bool variant_info(int variant, int arm, VariantInfo& v) {
  switch (variant) {
    case 1: CfgInfo<Cfg1>::get(arm, v); return true;
    case 2: CfgInfo<Cfg2>::get(arm, v); return true;
    case 3: CfgInfo<Cfg3>::get(arm, v); return true;
    case 4: CfgInfo<Cfg4>::get(arm, v); return true;
    case 5: CfgInfo<Cfg5>::get(arm, v); return true;
    case 6: CfgInfo<Cfg6>::get(arm, v); return true;
    case 7: CfgInfo<Cfg7>::get(arm, v); return true;
    case 8: CfgInfo<Cfg8>::get(arm, v); return true;
    case 9: CfgInfo<Cfg9>::get(arm, v); return true;
    case 10: CfgInfo<Cfg10>::get(arm, v); return true;
    case 11: CfgInfo<Cfg11>::get(arm, v); return true;
    default: return false;
  }
}

hipError_t launch_expert(int mode, int arm, int variant, int rung, const ExpertParams& p, int grid, int waves,
                         hipStream_t stream) {
  // the dequantize arm's MFMA pass reads dense weights and does not depend on the rung
  if (rung == kRungLut && arm != kArmDense) return launch_expert_lut(mode, arm, variant, p, grid, waves, stream);
  if (rung != kRungBitshift && rung != kRungLut) return hipErrorInvalidValue;
  return launch_expert_rung<kRungBitshift>(mode, arm, variant, p, grid, waves, stream);
}

hipError_t launch_pack_act(const uint16_t* x, const int32_t* padded_pair, const int32_t* n_pad, int32_t k,
                           int32_t H, int32_t n_pad_max, uint16_t* xs, hipStream_t stream) {
  const long items = (long)(n_pad_max >> 4) * (H / kKBlock) * 64;
  const long blocks = (items + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(pack_act_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, stream, x, padded_pair, n_pad, k, H,
                     n_pad_max, xs);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantParams& q, int rung, int grid, hipStream_t stream) {
  if (rung == kRungLut) return launch_dequant_lut(q, grid, stream);
  if (rung != kRungBitshift) return hipErrorInvalidValue;
  return launch_dequant_rung<kRungBitshift>(q, grid, stream);
}

hipError_t launch_combine(const float* y, const float* topk_w, int32_t n, int32_t k, int32_t H, void* out,
                          int out_bf16, hipStream_t stream) {
  const long total = (long)n * (H / 4);
  const int grid = (int)((total + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, stream, y, topk_w, n, k, H, out, out_bf16);
  return hipGetLastError();
}

hipError_t launch_gather_probe(int grid, int32_t rounds, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(gather_probe_kernel, dim3(grid), dim3(1024), 0, stream, rounds, sink);
  return hipGetLastError();
}

hipError_t launch_witness(int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(witness_kernel, dim3(1), dim3(1), 0, stream, out);
  return hipGetLastError();
}

}  // namespace qtip
