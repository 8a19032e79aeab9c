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
//    1024-thread workgroup per CU, persistent over wave-sized tasks.  Random 2-byte LUT
//    gathers are the decode's bottleneck, so LDS carries nothing else: decoded weights go
//    straight into MFMA B-operand registers instead of through an LDS weight tile, and
//    activations are read from global memory (L2-resident) into A-operand registers.
//  - A wave task is one unit (up to 64 binned pairs of one expert, i.e. several m-tiles
//    sharing one decode) x 16 output rows x all inputs.  Lane (j = lane%16, g = lane/16)
//    decodes row j; within each 128-input block lane group g owns the contiguous 32-symbol
//    run [32g, 32g+32), loaded as 8 bytes plus one look-ahead dword (the next 7 symbols,
//    wrapping to the row start at the row end: the window is circular).  The contraction
//    index is permuted accordingly: MFMA step s of a block pairs K slot 8g+t with input
//    32g + 8s + t, for both operands, which leaves the dot products unchanged.
//  - Grouped arm: v_mfma_f32_16x16x32_bf16 per 16-pair row block.  GEMV arm: the same
//    decoded registers feed VALU bf16 dot products per pair (8 pairs per decode).
#include "qtip_internal.h"

namespace qtip {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// fp16 -> bf16 bits: exact widening to fp32, then round to nearest even on the top 16 bits.
__device__ inline uint32_t f16_to_bf16_bits(uint32_t h) {
  const float f = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Stage the fp16 LUT into LDS as bf16 (8 entries per 16-byte load).
__device__ inline void fill_lut(uint16_t* lut_s, const uint16_t* __restrict__ lut_g) {
  const uint4* src = reinterpret_cast<const uint4*>(lut_g);
  uint4* dst = reinterpret_cast<uint4*>(lut_s);
  for (int i = threadIdx.x; i < kLutEntries / 8; i += blockDim.x) {
    const uint4 v = src[i];
    uint4 o;
    o.x = f16_to_bf16_bits(v.x & 0xFFFFu) | (f16_to_bf16_bits(v.x >> 16) << 16);
    o.y = f16_to_bf16_bits(v.y & 0xFFFFu) | (f16_to_bf16_bits(v.y >> 16) << 16);
    o.z = f16_to_bf16_bits(v.z & 0xFFFFu) | (f16_to_bf16_bits(v.z >> 16) << 16);
    o.w = f16_to_bf16_bits(v.w & 0xFFFFu) | (f16_to_bf16_bits(v.w >> 16) << 16);
    dst[i] = o;
  }
  __syncthreads();
}

__device__ inline uint32_t lut_pair(const uint16_t* lut, uint32_t s0, uint32_t s1) {
  return (uint32_t)lut[s0] | ((uint32_t)lut[s1] << 16);
}

// `win` holds 30 valid stream bits: bits [2t, 2t+16) are the state of symbol t, t = 0..7.
// Returns the 8 bf16 weights packed two per dword (symbol 2q low, 2q+1 high).
__device__ inline u32x4 decode8(const uint16_t* lut, uint32_t win) {
  u32x4 r;
  r[0] = lut_pair(lut, win & 0xFFFFu, (win >> 2) & 0xFFFFu);
  r[1] = lut_pair(lut, (win >> 4) & 0xFFFFu, (win >> 6) & 0xFFFFu);
  r[2] = lut_pair(lut, (win >> 8) & 0xFFFFu, (win >> 10) & 0xFFFFu);
  r[3] = lut_pair(lut, (win >> 12) & 0xFFFFu, (win >> 14) & 0xFFFFu);
  return r;
}

// Window of step s (symbols 8s..8s+7 of the lane's 32-symbol run): d0, d1 are the run's
// two dwords, la the look-ahead dword (the following 16 symbols).
__device__ inline uint32_t run_window(int s, uint32_t d0, uint32_t d1, uint32_t la) {
  switch (s) {
    case 0: return d0;
    case 1: return __builtin_amdgcn_alignbit(d1, d0, 16);
    case 2: return d1;
    default: return __builtin_amdgcn_alignbit(la, d1, 16);
  }
}

struct RunCodes {
  uint32_t d0, d1, la;
};

__device__ inline RunCodes load_run(const uint8_t* __restrict__ row, int ob, int row_bytes) {
  RunCodes rc;
  const uint2 v = *reinterpret_cast<const uint2*>(row + ob);
  int nx = ob + 8;
  if (nx >= row_bytes) nx -= row_bytes;
  rc.d0 = v.x;
  rc.d1 = v.y;
  rc.la = *reinterpret_cast<const uint32_t*>(row + nx);
  return rc;
}

// Takes the dword by value: __builtin_bit_cast applied directly to an ext-vector element
// (w[i]) compiles to a read of element 0 for every i with this clang, so each element is
// first copied into a plain uint32_t.
__device__ inline bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

__device__ inline float dot8(u32x4 w, u32x4 x, float acc) {
  const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
  const uint32_t x0 = x.x, x1 = x.y, x2 = x.z, x3 = x.w;
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(x0), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(x1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(x2), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(x3), acc, false);
  return acc;
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

struct Unit {
  int e, start, len;
};

// Reads and validates a unit; returns false for a unit that must be skipped.
__device__ inline bool read_unit(const ExpertParams& p, int u, Unit& un) {
  un.e = p.units[3 * u + 0];
  un.start = p.units[3 * u + 1];
  un.len = p.units[3 * u + 2];
  return un.e >= 0 && un.e < p.num_experts && un.len >= 1 && un.len <= kUnitMaxPairs && un.start >= 0 &&
         un.start <= p.n_pos - un.len;
}

// Activation row of binned position s, or -1 if it is out of range.
__device__ inline int act_row(const ExpertParams& p, int s) {
  int r = p.act_row_map ? p.act_row_map[s] / p.act_row_div : s;
  return (r >= 0 && r < p.n_act_rows) ? r : -1;
}

__device__ inline int out_row(const ExpertParams& p, int s) {
  int r = p.out_row_map ? p.out_row_map[s] : s;
  return (r >= 0 && r < p.n_out_rows) ? r : -1;
}

template <int MODE>
__device__ inline void epilogue_store(const ExpertParams& p, const Unit& un, int r, int pi, float a0, float a1,
                                      float s0, float s1) {
  const int s = un.start + pi;
  if (MODE == kModeGateUp) {
    const float g = a0 * s0, u = a1 * s1;
    const float h = silu(g) * u;
    reinterpret_cast<uint16_t*>(p.out)[(size_t)s * p.rows + r] = (uint16_t)f32_to_bf16_bits(h);
  } else {
    const int orow = out_row(p, s);
    if (orow >= 0) reinterpret_cast<float*>(p.out)[(size_t)orow * p.rows + r] = a0 * s0;
  }
}

template <int MODE>
__device__ void task_grouped(const ExpertParams& p, const uint16_t* lut, const Unit& un, int r0) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int r = r0 + j;
  const int row_bytes = p.cols >> 2;
  const int kblocks = p.cols / kKBlock;
  const uint8_t* row0 = p.codes0 + ((size_t)un.e * p.rows + r) * row_bytes;
  const uint8_t* row1 = (MODE == kModeGateUp) ? p.codes1 + ((size_t)un.e * p.rows + r) * row_bytes : nullptr;
  const int nsub = (un.len + 15) >> 4;

  // A operand rows of this lane (row i = lane%16 of each 16-pair block)
  const uint16_t* abase[4];
  bool aval[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int pi = m * 16 + j;
    int ar = (pi < un.len) ? act_row(p, un.start + pi) : -1;
    aval[m] = ar >= 0;
    abase[m] = p.act + (size_t)(ar >= 0 ? ar : 0) * p.cols + g * 32;
  }

  f32x4 acc0[4], acc1[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc0[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int kb = 0; kb < kblocks; ++kb) {
    const int ob = kb * 32 + g * 8;
    const RunCodes c0 = load_run(row0, ob, row_bytes);
    RunCodes c1{};
    if (MODE == kModeGateUp) c1 = load_run(row1, ob, row_bytes);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 b0 = decode8(lut, run_window(s, c0.d0, c0.d1, c0.la));
      u32x4 b1{};
      if (MODE == kModeGateUp) b1 = decode8(lut, run_window(s, c1.d0, c1.d1, c1.la));
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < nsub) {
          u32x4 a = u32x4{0u, 0u, 0u, 0u};
          if (aval[m]) a = *reinterpret_cast<const u32x4*>(abase[m] + kb * kKBlock + s * 8);
          acc0[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, b0), acc0[m], 0, 0, 0);
          if (MODE == kModeGateUp)
            acc1[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, b1), acc1[m], 0, 0, 0);
        }
      }
    }
  }

  // D layout: lane holds rows 4*(lane/16)+t (pairs) of column lane%16 (output row r)
  const float s0 = f16_to_f32(p.scale0[(size_t)un.e * p.rows + r]);
  const float s1 = (MODE == kModeGateUp) ? f16_to_f32(p.scale1[(size_t)un.e * p.rows + r]) : 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m < nsub) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pi = m * 16 + 4 * g + t;
        if (pi < un.len) epilogue_store<MODE>(p, un, r, pi, acc0[m][t], acc1[m][t], s0, s1);
      }
    }
  }
}

template <int MODE>
__device__ void task_gemv(const ExpertParams& p, const uint16_t* lut, const Unit& un, int r0) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int r = r0 + j;
  const int row_bytes = p.cols >> 2;
  const int kblocks = p.cols / kKBlock;
  const uint8_t* row0 = p.codes0 + ((size_t)un.e * p.rows + r) * row_bytes;
  const uint8_t* row1 = (MODE == kModeGateUp) ? p.codes1 + ((size_t)un.e * p.rows + r) * row_bytes : nullptr;
  const float s0 = f16_to_f32(p.scale0[(size_t)un.e * p.rows + r]);
  const float s1 = (MODE == kModeGateUp) ? f16_to_f32(p.scale1[(size_t)un.e * p.rows + r]) : 0.f;

  for (int q0 = 0; q0 < un.len; q0 += kGemvPairs) {
    const int nq = min(kGemvPairs, un.len - q0);
    const uint16_t* xb[kGemvPairs];
    bool xv[kGemvPairs];
#pragma unroll
    for (int q = 0; q < kGemvPairs; ++q) {
      const int ar = (q < nq) ? act_row(p, un.start + q0 + q) : -1;
      xv[q] = ar >= 0;
      xb[q] = p.act + (size_t)(ar >= 0 ? ar : 0) * p.cols + g * 32;
    }
    float acc0[kGemvPairs], acc1[kGemvPairs];
#pragma unroll
    for (int q = 0; q < kGemvPairs; ++q) acc0[q] = acc1[q] = 0.f;

    for (int kb = 0; kb < kblocks; ++kb) {
      const int ob = kb * 32 + g * 8;
      const RunCodes c0 = load_run(row0, ob, row_bytes);
      RunCodes c1{};
      if (MODE == kModeGateUp) c1 = load_run(row1, ob, row_bytes);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 b0 = decode8(lut, run_window(s, c0.d0, c0.d1, c0.la));
        u32x4 b1{};
        if (MODE == kModeGateUp) b1 = decode8(lut, run_window(s, c1.d0, c1.d1, c1.la));
#pragma unroll
        for (int q = 0; q < kGemvPairs; ++q) {
          if (q < nq && xv[q]) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(xb[q] + kb * kKBlock + s * 8);
            acc0[q] = dot8(b0, x, acc0[q]);
            if (MODE == kModeGateUp) acc1[q] = dot8(b1, x, acc1[q]);
          }
        }
      }
    }
    // sum the four lane groups (lanes j, j+16, j+32, j+48 hold one row's partial sums)
#pragma unroll
    for (int q = 0; q < kGemvPairs; ++q) {
      float a0 = acc0[q];
      a0 += __shfl_xor(a0, 16, 64);
      a0 += __shfl_xor(a0, 32, 64);
      float a1 = 0.f;
      if (MODE == kModeGateUp) {
        a1 = acc1[q];
        a1 += __shfl_xor(a1, 16, 64);
        a1 += __shfl_xor(a1, 32, 64);
      }
      if (q < nq && (q & 3) == g) epilogue_store<MODE>(p, un, r, q0 + q, a0, a1, s0, s1);
    }
  }
}

template <int MODE, int ARM>
__global__ __launch_bounds__(kExpertThreads, 1) void expert_kernel(ExpertParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lut_s[kLutEntries];
  fill_lut(lut_s, p.lut);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = p.n_units_dev ? __builtin_amdgcn_readfirstlane(*p.n_units_dev) : p.n_units_host;
  const int nblocks = p.rows / kRowsPerTask;
  const long total = (long)n_units * nblocks;
  const long stride = (long)gridDim.x * kExpertWaves;
  for (long task = (long)blockIdx.x * kExpertWaves + wave; task < total; task += stride) {
    const int u = (int)(task / nblocks);
    const int nb = (int)(task - (long)u * nblocks);
    Unit un;
    if (!read_unit(p, u, un)) continue;
    if (ARM == kArmGrouped)
      task_grouped<MODE>(p, lut_s, un, nb * kRowsPerTask);
    else
      task_gemv<MODE>(p, lut_s, un, nb * kRowsPerTask);
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
  for (int jj = 0; jj < k; ++jj) {
    const float wt = w[(size_t)t * k + jj];
    const float4 v = *reinterpret_cast<const float4*>(y + ((size_t)t * k + jj) * H + c);
    acc.x = fmaf(wt, v.x, acc.x);
    acc.y = fmaf(wt, v.y, acc.y);
    acc.z = fmaf(wt, v.z, acc.z);
    acc.w = fmaf(wt, v.w, acc.w);
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

}  // namespace

hipError_t launch_expert(int mode, int arm, const ExpertParams& p, int grid, hipStream_t stream) {
  const dim3 g(grid), b(kExpertThreads);
  if (mode == kModeGateUp && arm == kArmGrouped)
    hipLaunchKernelGGL((expert_kernel<kModeGateUp, kArmGrouped>), g, b, 0, stream, p);
  else if (mode == kModeGateUp)
    hipLaunchKernelGGL((expert_kernel<kModeGateUp, kArmGemv>), g, b, 0, stream, p);
  else if (arm == kArmGrouped)
    hipLaunchKernelGGL((expert_kernel<kModeSingle, kArmGrouped>), g, b, 0, stream, p);
  else
    hipLaunchKernelGGL((expert_kernel<kModeSingle, kArmGemv>), g, b, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* topk_w, int32_t n, int32_t k, int32_t H, void* out,
                          int out_bf16, hipStream_t stream) {
  const long total = (long)n * (H / 4);
  const int grid = (int)((total + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, stream, y, topk_w, n, k, H, out, out_bf16);
  return hipGetLastError();
}

hipError_t launch_witness(int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(witness_kernel, dim3(1), dim3(1), 0, stream, out);
  return hipGetLastError();
}

}  // namespace qtip
