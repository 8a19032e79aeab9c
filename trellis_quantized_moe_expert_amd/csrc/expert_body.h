// Expert-kernel templates shared by the two rungs' translation units (expert.hip: the bitshift
// rung and the rung-independent kernels; expert_lut.hip: the LUT rung).  Not part of the ABI.
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
//  - The decoder's table lives in LDS; one workgroup of 8, 12 or 16 waves per CU, persistent over
//    wave-sized tasks.  Bitshift rung: the 65536-entry LUT narrowed to bf16 (128 KiB of the
//    160 KiB); its random 2-byte gathers are the decode's bottleneck, so decoded weights go
//    straight into MFMA B-operand registers instead of through an LDS weight tile, and
//    activations are read from global memory (L2-resident) into A-operand registers.  LUT rung:
//    the 512 x 2 codebook as 32 bank-replicated copies (64 KiB), one conflict-free read per two
//    weights; that rung waits on its vector-memory loads instead, so its loops load codes
//    transposed and pipeline them (DecoderLut::kPipelined).  (Small GEMV launches also keep
//    partial sums in the rest of LDS; see gemv_split_tasks.)
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
#pragma once

#include <type_traits>

#include "qtip_internal.h"
#include "route_device.h"

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

__device__ inline uint32_t lut_bf16x2(uint32_t v) {
  return f16_to_bf16_bits(v & 0xFFFFu) | (f16_to_bf16_bits(v >> 16) << 16);
}

// Stage the fp16 LUT into LDS as bf16 (8 entries per 16-byte load) with a workgroup of THREADS
// threads: every load of a thread is issued before the first conversion, so the fill waits for
// one memory round trip instead of one per load.
template <int THREADS>
__device__ inline void fill_lut(uint16_t* lut_s, const uint16_t* __restrict__ lut_g) {
  constexpr int kVec = kLutEntries / 8;
  constexpr int kIter = (kVec + THREADS - 1) / THREADS;
  const uint4* src = reinterpret_cast<const uint4*>(lut_g);
  uint4* dst = reinterpret_cast<uint4*>(lut_s);
  uint4 v[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int i = (int)threadIdx.x + it * THREADS;
    if (kVec % THREADS == 0 || i < kVec) v[it] = src[i];
  }
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int i = (int)threadIdx.x + it * THREADS;
    if (kVec % THREADS == 0 || i < kVec)
      dst[i] = uint4{lut_bf16x2(v[it].x), lut_bf16x2(v[it].y), lut_bf16x2(v[it].z), lut_bf16x2(v[it].w)};
  }
  __syncthreads();
}

// The same with any workgroup size (a launch with fewer waves than its configuration's), four
// loads of a thread in flight at a time (measured: sixteen made the one-token down pass slower).
__device__ inline void fill_lut_any(uint16_t* lut_s, const uint16_t* __restrict__ lut_g) {
  constexpr int kVec = kLutEntries / 8;
  constexpr int kBatch = 4;
  const uint4* src = reinterpret_cast<const uint4*>(lut_g);
  uint4* dst = reinterpret_cast<uint4*>(lut_s);
  for (int i0 = 0; i0 < kVec; i0 += kBatch * (int)blockDim.x) {
    uint4 v[kBatch];
#pragma unroll
    for (int it = 0; it < kBatch; ++it) {
      const int i = i0 + (int)threadIdx.x + it * (int)blockDim.x;
      if (i < kVec) v[it] = src[i];
    }
#pragma unroll
    for (int it = 0; it < kBatch; ++it) {
      const int i = i0 + (int)threadIdx.x + it * (int)blockDim.x;
      if (i < kVec) dst[i] = uint4{lut_bf16x2(v[it].x), lut_bf16x2(v[it].y), lut_bf16x2(v[it].z), lut_bf16x2(v[it].w)};
    }
  }
  __syncthreads();
}

__device__ inline uint32_t lut_pair(const uint16_t* lut, uint32_t s0, uint32_t s1) {
  return (uint32_t)lut[s0] | ((uint32_t)lut[s1] << 16);
}

// Decode 16 consecutive symbols of a run.  `lo` holds the stream bits of the 16 symbols,
// `hi` the 16 symbols after them (the look-ahead).  The 32-bit window alignbit(hi, lo, 2t)
// holds the state of symbol t in its low half and of symbol t+8 in its high half, so one
// funnel shift serves two symbols.  Returns the 8 bf16 weights of symbols 0..7 in `first`
// and of symbols 8..15 in `second`, packed two per dword (lower symbol in the low half).
__device__ inline void decode16(const uint16_t* lut, uint32_t lo, uint32_t hi, u32x4& first, u32x4& second) {
  uint32_t x[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) x[t] = (t == 0) ? lo : __builtin_amdgcn_alignbit(hi, lo, 2 * t);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    first[q] = lut_pair(lut, x[2 * q] & 0xFFFFu, x[2 * q + 1] & 0xFFFFu);
    second[q] = lut_pair(lut, x[2 * q] >> 16, x[2 * q + 1] >> 16);
  }
}

// Decoders of one 16-symbol piece of a run, one per rung; `decode16` has the same contract for
// both: 8 bf16 weights of symbols 0..7 in `first`, of symbols 8..15 in `second`, two per dword.
// kPipelined selects the block loop.  The bitshift rung is bound by its LDS gathers, which hide
// memory latency and leave no LDS time for cross-lane moves: its loops load codes directly in the
// MFMA layout, one block ahead.  The LUT rung's gathers are cheap, and its loops are bound by the
// vector-memory path instead: they load codes transposed (to_mfma_layout) and run over ping-pong
// buffers so that the one-block prefetch survives compilation.
struct DecoderBitshift {
  static constexpr bool kPipelined = false;
  const uint16_t* lut;  // the bf16 LUT in LDS (65536 entries)
  __device__ inline void decode16(uint32_t lo, uint32_t hi, u32x4& first, u32x4& second) const {
    ::qtip::decode16(lut, lo, hi, first, second);
  }
};

// LUT rung: the codebook in LDS as 32 copies of each entry, the entry's bf16 pair in one dword,
// entry s's copy c at dword 32 s + c.  Lane l reads copy l % 32, so the 32 lanes of a half-wave
// always read 32 different banks: the gathers never conflict, and each returns two weights.
// Pair states sit at even symbols: the window alignbit(hi, lo, 4q) holds the state of the pair at
// symbol 2q in its low 9 bits and of the pair at symbol 2q + 8 in bits 16..24.
struct DecoderLut {
  static constexpr bool kPipelined = true;
  const char* cb;     // LDS codebook, 32 x 4 bytes per entry
  uint32_t bank_off;  // (lane % 32) * 4
  __device__ inline uint32_t entry(uint32_t byte_off) const {
    return *reinterpret_cast<const uint32_t*>(cb + byte_off);
  }
  __device__ inline void decode16(uint32_t lo, uint32_t hi, u32x4& first, u32x4& second) const {
    uint32_t x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = (q == 0) ? lo : __builtin_amdgcn_alignbit(hi, lo, 4 * q);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      first[q] = entry(((x[q] & (uint32_t)(kCodebookEntries - 1)) << 7) | bank_off);
      second[q] = entry(((x[q] >> 9) & ((uint32_t)(kCodebookEntries - 1) << 7)) | bank_off);
    }
  }
};

// Stage the fp16 codebook [512][2] into LDS as bf16 pairs, 32 copies per entry (DecoderLut): each
// thread converts one entry and writes 4 of its copies with one 16-byte store.
__device__ inline void fill_codebook(uint32_t* cb_s, const uint16_t* __restrict__ cb_g) {
  const uint32_t* src = reinterpret_cast<const uint32_t*>(cb_g);
  uint4* dst = reinterpret_cast<uint4*>(cb_s);
  constexpr int kStores = kCodebookEntries * kCodebookCopies / 4;
  for (int i = (int)threadIdx.x; i < kStores; i += (int)blockDim.x) {
    const uint32_t v = lut_bf16x2(src[i / (kCodebookCopies / 4)]);
    dst[i] = uint4{v, v, v, v};
  }
  __syncthreads();
}

struct RunCodes {
  uint32_t d0, d1, la;
};

// Codes are loaded transposed: lane 4r + c loads chunk c (8 bytes, plus its 4-byte look-ahead) of
// row r of the task's 16-row block, so the four lanes of each quad read one row's consecutive
// bytes, and with the LUT rung's block-interleaved layout a wave's 16 rows x 32 bytes of a block
// are 512 contiguous bytes (four lines, instead of sixteen in a row-major layout).  The MFMA operand
// layout wants chunk g
// of row j in lane j + 16g; one cross-lane pull per dword (ds_bpermute: lane L reads lane
// 4 (L % 16) + L / 16) moves the loaded dwords there before the decode.
__device__ inline int code_row(int lane) { return lane >> 2; }
__device__ inline int code_chunk(int lane) { return lane & 3; }
__device__ inline RunCodes to_mfma_layout(const RunCodes& t) {
  const int lane = threadIdx.x & 63;
  const int addr = (((lane & 15) << 2) | (lane >> 4)) << 2;
  return RunCodes{(uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)t.d0),
                  (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)t.d1),
                  (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)t.la)};
}

// A run's 8 bytes without the look-ahead (the grouped arm's descending loop takes the look-ahead
// from the neighbouring run instead), transposed like RunCodes.
struct RunChunk {
  uint32_t d0, d1;
};
template <int NT>
struct ChunkSet {
  RunChunk c[NT];
};
template <int NT>
__device__ inline ChunkSet<NT> load_chunks(const uint8_t* __restrict__ base, uint32_t row_off0, uint32_t nt_stride,
                                           int ob) {
  ChunkSet<NT> cs;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint2 v = *reinterpret_cast<const uint2*>(base + (row_off0 + nt * nt_stride + (uint32_t)ob));
    cs.c[nt] = RunChunk{v.x, v.y};
  }
  return cs;
}
// Lane j+16g gets chunk g of row j: d0, d1 pulled from the transposed lanes, and the look-ahead
// from lane j+16(g+1), the next chunk's d0; lane group 3 reads lane group 0, whose `prev` (the
// first dword of the row's next block, already in MFMA layout) it gets instead.
__device__ inline RunCodes chunk_to_mfma_layout(const RunChunk& t, uint32_t prev, int cv_addr, int la_addr, int g) {
  RunCodes r;
  r.d0 = (uint32_t)__builtin_amdgcn_ds_bpermute(cv_addr, (int)t.d0);
  r.d1 = (uint32_t)__builtin_amdgcn_ds_bpermute(cv_addr, (int)t.d1);
  r.la = (uint32_t)__builtin_amdgcn_ds_bpermute(la_addr, (int)(g == 0 ? prev : r.d0));
  return r;
}

// Codes are stored block-interleaved: the 16 rows x 32 bytes of one 16-row block and one
// 128-input block lie together (512 bytes, the blocks of a 16-row block consecutive), so a wave's
// loads of a block touch four whole 128-byte lines, each used once.  Row r's bytes [32 kb, 32 kb +
// 32) sit at byte ((r / 16) kblocks + kb) 512 + (r % 16) 32 of its matrix: row r's offset is
// code_blk_row(r), block kb's kCodeBlk * kb.  `base` is the (wave-uniform) start of the expert's
// matrix; 32-bit offsets keep the addresses in one VGPR each.
constexpr int kCodeBlk = 512;
// Dequantize arm: blocks whose codes are requested together, ahead of the previous ones' stores.
constexpr int kDqBatch = 4;
__device__ inline uint32_t code_blk_row(int r, int row_bytes) {
  return (uint32_t)(r >> 4) * (16u * (uint32_t)row_bytes) + (uint32_t)(r & 15) * 32u;
}

// A run (chunk tc of block kb) in the block-interleaved layout: 8 bytes, and the look-ahead
// dword, which is the next chunk's first dword, or for chunk 3 the first dword of block kb + 1
// (of block 0 after the row's last block: the window is circular).
__device__ inline RunCodes load_run_blk(const uint8_t* __restrict__ base, uint32_t row_off, int kb, int tc,
                                        int kblocks) {
  const uint32_t o = row_off + (uint32_t)(kb * kCodeBlk + tc * 8);
  const uint32_t la = tc < 3 ? o + 8u : row_off + (uint32_t)((kb + 1 < kblocks ? kb + 1 : 0) * kCodeBlk);
  const uint2 v = *reinterpret_cast<const uint2*>(base + o);
  RunCodes rc;
  rc.d0 = v.x;
  rc.d1 = v.y;
  rc.la = *reinterpret_cast<const uint32_t*>(base + la);
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
  int pad;  // start in the padded position space (a multiple of 16), or -1 without one
};

// Reads and validates a unit; returns false for a unit that must be skipped.
__device__ inline bool read_unit(const ExpertParams& p, int u, Unit& un) {
  un.e = p.units[3 * u + 0];
  un.start = p.units[3 * u + 1];
  un.len = p.units[3 * u + 2];
  un.pad = p.unit_pad ? p.unit_pad[u] : -1;
  const bool pad_ok = !p.unit_pad || (un.pad >= 0 && (un.pad & 15) == 0 && un.pad <= p.n_pad_max - ((un.len + 15) & ~15));
  return un.e >= 0 && un.e < p.num_experts && un.len >= 1 && un.len <= kUnitMaxPairs && un.start >= 0 &&
         un.start <= p.n_pos - un.len && pad_ok;
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
                                      float s0, float s1, int orow) {
  const int s = un.start + pi;
  if (MODE == kModeGateUp) {
    const float g = a0 * s0, u = a1 * s1;
    const float h = silu(g) * u;
    size_t o;
    if (p.unit_pad) {
      // h in fragment order over padded positions, as the down pass reads its A operand
      // (its input index r = kb*128 + 32g + 8st + t)
      const int pp = un.pad + pi;
      o = dense_fragment_offset(pp >> 4, r >> 7, (r >> 3) & 3, (pp & 15) + 16 * ((r >> 5) & 3), p.rows >> 7) + (r & 7);
    } else {
      o = (size_t)s * p.rows + r;
    }
    reinterpret_cast<uint16_t*>(p.out)[o] = (uint16_t)f32_to_bf16_bits(h);
  } else {
    // orow: out_row(p, s), loaded when the task started
    if (orow >= 0) reinterpret_cast<float*>(p.out)[(size_t)orow * p.rows + r] = a0 * s0;
  }
}

// Activation loads go through a buffer resource whose range ends at 2^31 bytes.  The plan keeps
// every activation buffer below 2^30 elements, so each real fragment lies inside the range; a
// lane whose row is past its unit gets the element offset kNoActRow (byte offset 2^31), and its
// load returns zeros without a memory access.  The instruction still counts as one load for the
// whole wave (no branch, so the compiler counts outstanding memory operations exactly), while
// the lanes it skips cost no cache access.  Only the MFMA output row of such a lane reads the
// zeros (each output row depends on its own A row alone), and that row is never stored.
constexpr uint32_t kNoActRow = 1u << 30;
constexpr uint32_t kActRangeBytes = 1u << 31;

__device__ inline __amdgpu_buffer_rsrc_t act_rsrc(const uint16_t* act) {
  // raw buffer (stride 0), range in bytes; the last word is the gfx9 data format for untyped loads
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(act), (short)0, (int)kActRangeBytes, 0x00020000);
}

// 16 bytes at byte offset voff + soff (soff wave-uniform, the position within a row); a voff at
// or past kActRangeBytes reads zeros.  voff + soff stays below 2^32: soff is below a row's bytes.
__device__ inline u32x4 act_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)soff, 0));
}

// Loads the A fragments of one K block: for each 16-pair row block m < NS, the 16 bytes of
// each of the 4 MFMA steps (K slots 8g..8g+7 <-> inputs kb*128 + 32g + 8s + 0..7).
template <int NS>
__device__ inline void load_a_block(u32x4 (&a)[NS][4], const uint16_t* __restrict__ act, const uint32_t (&aoff)[NS],
                                    int kb) {
  const __amdgpu_buffer_rsrc_t rs = act_rsrc(act);
#pragma unroll
  for (int m = 0; m < NS; ++m) {
#pragma unroll
    for (int st = 0; st < 4; ++st) a[m][st] = act_load16(rs, aoff[m] * 2u, (uint32_t)(kb * kKBlock * 2 + st * 16));
  }
}

// The same fragments from activations in fragment order: for 16-pair block m the wave's 64
// lanes read 1 KiB contiguous per MFMA step (fo[m] = the block's offset for this lane at kb = 0,
// st = 0; consecutive steps are 512 elements apart, blocks 2048).
template <int NS>
__device__ inline void load_a_block_frag(u32x4 (&a)[NS][4], const uint16_t* __restrict__ act, const uint32_t (&fo)[NS],
                                         int kb) {
  const __amdgpu_buffer_rsrc_t rs = act_rsrc(act);
#pragma unroll
  for (int m = 0; m < NS; ++m) {
#pragma unroll
    for (int st = 0; st < 4; ++st) a[m][st] = act_load16(rs, fo[m] * 2u, (uint32_t)(kb * 4096 + st * 1024));
  }
}

template <int NS, bool FRAG>
__device__ inline void load_a(u32x4 (&a)[NS][4], const uint16_t* __restrict__ act, const uint32_t (&off)[NS], int kb) {
  if (FRAG) load_a_block_frag<NS>(a, act, off, kb);
  else load_a_block<NS>(a, act, off, kb);
}

// Activation row offsets (elements from p.act) of this lane for NS entries; entry m is the
// binned position first + m*stride.  Positions past the unit, and rows out of range, get
// kNoActRow: their loads read zeros, and their results are never stored.
template <int NS>
__device__ inline void act_rows(const ExpertParams& p, const Unit& un, int first, int stride, int g,
                                uint32_t (&off)[NS]) {
#pragma unroll
  for (int m = 0; m < NS; ++m) {
    const int pi = first + m * stride;
    const int ar = (pi < un.len) ? act_row(p, un.start + pi) : -1;
    off[m] = ar >= 0 ? (uint32_t)ar * (uint32_t)p.cols + (uint32_t)(g * 32) : kNoActRow;
  }
}

// Codes of one 32-symbol run for each of NT row blocks (rows r0 + 16*nt + j).
template <int NT>
struct RunSet {
  RunCodes c[NT];
};

// The prefetch loops below carry a value loaded before the loop (the first block's codes or
// activations) that each iteration replaces by a load for the next block.  Left alone, the
// compiler merges those two loads into one load of a merged address at the top of the loop body,
// which then waits for its own data: the one-block prefetch disappears and every block waits a
// full memory round trip.  Passing the values loaded before the loop through an empty asm (no
// instruction, registers only) makes them opaque, so the loads stay where the loop puts them.
__device__ inline void keep_apart(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ inline void keep_apart(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ inline void keep_apart(RunCodes& c) {
  keep_apart(c.d0);
  keep_apart(c.d1);
  keep_apart(c.la);
}
template <int NT>
__device__ inline void keep_apart(RunSet<NT>& r) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) keep_apart(r.c[nt]);
}
template <int NT>
__device__ inline void keep_apart(ChunkSet<NT>& r) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    keep_apart(r.c[nt].d0);
    keep_apart(r.c[nt].d1);
  }
}
template <int NS>
__device__ inline void keep_apart(u32x4 (&a)[NS][4]) {
#pragma unroll
  for (int m = 0; m < NS; ++m) {
#pragma unroll
    for (int st = 0; st < 4; ++st) keep_apart(a[m][st]);
  }
}

template <int NT>
__device__ inline RunSet<NT> to_mfma_layout(const RunSet<NT>& t) {
  RunSet<NT> r;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) r.c[nt] = to_mfma_layout(t.c[nt]);
  return r;
}

// The look-ahead dwords alone (see load_run_blk), for NT row blocks.
template <int NT>
__device__ inline void load_las_blk(uint32_t (&la)[NT], const uint8_t* __restrict__ base, uint32_t row_off0,
                                    uint32_t nt_stride, int kb, int tc, int kblocks) {
  const uint32_t o = tc < 3 ? (uint32_t)(kb * kCodeBlk + tc * 8 + 8) : (uint32_t)((kb + 1 < kblocks ? kb + 1 : 0) * kCodeBlk);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) la[nt] = *reinterpret_cast<const uint32_t*>(base + (row_off0 + nt * nt_stride + o));
}

template <int NT>
__device__ inline RunSet<NT> load_runs_blk(const uint8_t* __restrict__ base, uint32_t row_off0, uint32_t nt_stride,
                                           int kb, int tc, int kblocks) {
  RunSet<NT> rs;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) rs.c[nt] = load_run_blk(base, row_off0 + nt * nt_stride, kb, tc, kblocks);
  return rs;
}

// Block order of a task (the bitshift rung's loops and the dequantize arm): a row's last 128-input
// block first (the one whose look-ahead wraps to the row's first block, loaded before the loop),
// then blocks 0, 1, ..., kblocks-2.  Iteration i works on block_at(i) and prefetches block_at(i +
// 1) = i; the last iteration's prefetch (block 0) is not used.
__device__ inline int block_at(int i, int kblocks) { return i == 0 ? kblocks - 1 : i - 1; }

// Grouped and dequantize arms: scale and store one task's 16-pair x 16-row MFMA tiles.
// What the single-matrix pass's epilogue reads from memory, requested when the task starts so
// that the loads are not a round trip of their own after the last block (there the output row
// is a dependent lookup through the binned order): lane i holds the scale of the task's row
// r0 + i (i < 16 NT <= 64) and the output row of the unit's pair i (i < len <= 64); the epilogue
// moves them across lanes.  The fused pass loads its two scales in the epilogue (prefetching
// them measured no gain there and costs registers its kernels do not have).
struct EpiPre {
  float s0;
  int orow;
};

template <int MODE, int NT>
__device__ inline EpiPre epilogue_prefetch(const ExpertParams& p, const Unit& un, int r0) {
  const int lane = threadIdx.x & 63;
  EpiPre e{0.f, -1};
  if constexpr (MODE == kModeSingle) {
    if (lane < 16 * NT) e.s0 = f16_to_f32(p.scale0[(size_t)un.e * p.rows + r0 + lane]);
    if (lane < un.len) e.orow = out_row(p, un.start + lane);
  }
  return e;
}

// D layout: lane holds rows 4*(lane/16)+t (pairs) of column lane%16 (output row).
template <int MODE, int NS, int NT>
__device__ inline void grouped_epilogue(const ExpertParams& p, const Unit& un, int r0, const f32x4 (&acc0)[NS][NT],
                                        const f32x4 (&acc1)[NS][NT], const EpiPre& pre) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + 16 * nt + j;
    const float s0 = (MODE == kModeSingle) ? __shfl(pre.s0, 16 * nt + j, 64)
                                           : f16_to_f32(p.scale0[(size_t)un.e * p.rows + r]);
    const float s1 = (MODE == kModeGateUp) ? f16_to_f32(p.scale1[(size_t)un.e * p.rows + r]) : 0.f;
#pragma unroll
    for (int m = 0; m < NS; ++m) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pi = m * 16 + 4 * g + t;
        const int orow = (MODE == kModeSingle) ? __shfl(pre.orow, pi & 63, 64) : -1;
        if (pi < un.len) epilogue_store<MODE>(p, un, r, pi, acc0[m][nt][t], acc1[m][nt][t], s0, s1, orow);
      }
    }
  }
}

// The dense-weight slot of woken expert e: the number of experts below e with binned pairs (the
// woken experts are materialised compactly, so the workspace holds min(E, n k) of them).  Every
// lane of the wave gets the same value.
__device__ inline int dense_slot(const int32_t* __restrict__ counts, int e) {
  const int lane = threadIdx.x & 63;
  int c = 0;
  for (int i = lane; i < e; i += 64) c += counts[i] > 0 ? 1 : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  return __builtin_amdgcn_readfirstlane(c);
}

// Number of experts with pairs (wave-uniform).
__device__ inline int woken_count(const int32_t* __restrict__ counts, int E) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (int b = 0; b < E; b += 64) n += __popcll(__ballot(b + lane < E && counts[b + lane] > 0));
  return __builtin_amdgcn_readfirstlane(n);
}

// The expert with pairs at slot s (the s-th in ascending expert order), or -1 past the last.
__device__ inline int nth_woken(const int32_t* __restrict__ counts, int E, int s) {
  const int lane = threadIdx.x & 63;
  int below = 0;
  for (int b = 0; b < E; b += 64) {
    const bool v = b + lane < E && counts[b + lane] > 0;
    const uint64_t m = __ballot(v);
    const int pc = __popcll(m);
    if (s < below + pc) {
      const int before = __popcll(m & ((1ull << lane) - 1ull));  // woken lanes below this one
      const uint64_t hit = __ballot(v && before == s - below);
      return b + (int)__builtin_ctzll(hit);
    }
    below += pc;
  }
  return -1;
}

// Dequantize arm: the grouped pass over weights materialised beforehand as dense bf16 in
// fragment order (no decode, no LUT): the B fragment of MFMA step st of block kb for row
// block r0/16 + nt is one coalesced 16-byte load per lane.  Same K permutation as the decode.
template <int MODE, int NS, int NT>
__device__ void task_dense(const ExpertParams& p, const Unit& un, int r0) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int kblocks = p.cols / kKBlock;
  const size_t mat = (size_t)p.rows * (size_t)p.cols;
  const size_t slot = (size_t)dense_slot(p.dense_counts, un.e);
  const uint16_t* w0 = p.dense0 + slot * mat;
  const uint16_t* w1 = (MODE == kModeGateUp) ? p.dense1 + slot * mat : w0;
  const int rb0 = r0 / 16;
  const EpiPre pre = epilogue_prefetch<MODE, NT>(p, un, r0);

  uint32_t aoff[NS];
  act_rows<NS>(p, un, j, 16, g, aoff);
  f32x4 acc0[NS][NT], acc1[NS][NT];
#pragma unroll
  for (int m = 0; m < NS; ++m) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc0[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int kb = 0; kb < kblocks; ++kb) {
    u32x4 a[NS][4];
    load_a_block<NS>(a, p.act, aoff, kb);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const size_t o = dense_fragment_offset(rb0 + nt, kb, st, lane, kblocks);
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(w0 + o);
        const u32x4 b1 = (MODE == kModeGateUp) ? *reinterpret_cast<const u32x4*>(w1 + o) : b0;
#pragma unroll
        for (int m = 0; m < NS; ++m) {
          acc0[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[m][st]),
                                                                __builtin_bit_cast(bf16x8, b0), acc0[m][nt], 0, 0, 0);
          if (MODE == kModeGateUp)
            acc1[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[m][st]),
                                                                  __builtin_bit_cast(bf16x8, b1), acc1[m][nt], 0, 0, 0);
        }
      }
    }
  }
  grouped_epilogue<MODE, NS, NT>(p, un, r0, acc0, acc1, pre);
}

// Grouped arm: NS row blocks of 16 pairs x NT row blocks of 16 outputs share one decode of
// the 16*NT rows; each A fragment feeds NT MFMAs.
template <int MODE, int NS, int NT, bool APRE, bool FRAG = false, class DEC = DecoderBitshift>
__device__ void task_grouped(const ExpertParams& p, const DEC& lut, const Unit& un, int r0) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int row_bytes = p.cols >> 2;
  const int kblocks = p.cols / kKBlock;
  // matrix bases are wave-uniform; each lane's row is a 32-bit byte offset from them
  const size_t mat_bytes = (size_t)p.rows * row_bytes;
  const uint8_t* base0 = p.codes0 + (size_t)un.e * mat_bytes;
  const uint8_t* base1 = (MODE == kModeGateUp) ? p.codes1 + (size_t)un.e * mat_bytes : base0;
  // this lane's code chunk and row: transposed for a pipelined decoder (LUT rung, block-interleaved
  // codes), the MFMA layout otherwise
  const int tc = DEC::kPipelined ? code_chunk(lane) : g;
  const uint32_t roff = code_blk_row(r0 + (DEC::kPipelined ? code_row(lane) : j), row_bytes);
  const uint32_t nt_stride = 16u * (uint32_t)row_bytes;
  const EpiPre pre = epilogue_prefetch<MODE, NT>(p, un, r0);

  uint32_t aoff[NS];  // A operand row i = lane%16 of each 16-pair block
  if (FRAG) {
#pragma unroll
    for (int m = 0; m < NS; ++m)
      aoff[m] = 16 * m + j < un.len ? (uint32_t)dense_fragment_offset((un.pad >> 4) + m, 0, 0, lane, kblocks) : kNoActRow;
  } else {
    act_rows<NS>(p, un, j, 16, g, aoff);
  }

  f32x4 acc0[NS][NT], acc1[NS][NT];
#pragma unroll
  for (int m = 0; m < NS; ++m) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc0[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  if constexpr (!DEC::kPipelined) {
    // Per block: the block's activations are requested first, then the next block's codes
    // (the block after the last wraps to block 0 and is not used), so waiting for the
    // activations never waits for those codes (memory counters retire in order) and the
    // codes have the whole block's decode to arrive.
    // With APRE the activations are double-buffered as well: block kb+1's are requested during
    // block kb, so every wait in the loop is for loads issued a whole block earlier.
    u32x4 an[NS][4];
    if (APRE) load_a<NS, FRAG>(an, p.act, aoff, kblocks - 1);
    RunSet<NT> n0 = load_runs_blk<NT>(base0, roff, nt_stride, kblocks - 1, tc, kblocks);
    RunSet<NT> n1 = (MODE == kModeGateUp) ? load_runs_blk<NT>(base1, roff, nt_stride, kblocks - 1, tc, kblocks) : n0;
    for (int i = 0; i < kblocks; ++i) {
      const int kb = block_at(i, kblocks);
      const int kn = i + 1 < kblocks ? i : 0;  // block_at(i + 1); unused after the last block
      u32x4 a[NS][4];
      if (APRE) {
#pragma unroll
        for (int m = 0; m < NS; ++m) {
#pragma unroll
          for (int st = 0; st < 4; ++st) a[m][st] = an[m][st];
        }
        load_a<NS, FRAG>(an, p.act, aoff, kn);
      } else {
        load_a<NS, FRAG>(a, p.act, aoff, kb);
      }
      const RunSet<NT> c0 = n0, c1 = n1;
      n0 = load_runs_blk<NT>(base0, roff, nt_stride, kn, tc, kblocks);
      if (MODE == kModeGateUp) n1 = load_runs_blk<NT>(base1, roff, nt_stride, kn, tc, kblocks);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          u32x4 b0[2], b1[2];
          const RunCodes& x0 = c0.c[nt];
          lut.decode16(h ? x0.d1 : x0.d0, h ? x0.la : x0.d1, b0[0], b0[1]);
          if (MODE == kModeGateUp) {
            const RunCodes& x1 = c1.c[nt];
            lut.decode16(h ? x1.d1 : x1.d0, h ? x1.la : x1.d1, b1[0], b1[1]);
          }
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const int st = 2 * h + hs;
#pragma unroll
            for (int m = 0; m < NS; ++m) {
              acc0[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[m][st]),
                                                                    __builtin_bit_cast(bf16x8, b0[hs]), acc0[m][nt], 0, 0, 0);
              if (MODE == kModeGateUp)
                acc1[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[m][st]),
                                                                      __builtin_bit_cast(bf16x8, b1[hs]), acc1[m][nt], 0, 0, 0);
            }
          }
        }
      }
    }
  } else {
    // Blocks in descending order, kblocks-1 down to 0, over ping-pong buffers (A, B) unrolled by
    // two: per block the activations are requested first, then the next block's codes (8 bytes
    // per lane, one 32-byte sector per row; the load after block 0 repeats block 0 and is not
    // used), so every wait is for loads issued a whole block earlier and no register copy
    // (which would wait for the load it copies) is needed between blocks.
    // A run's look-ahead is the first dword of the next run of its row: for chunks 0-2 the
    // next chunk's first dword in the same block, for chunk 3 the first dword of block kb+1,
    // which descending order has just decoded (its MFMA-layout d0 is carried from the previous
    // block); the first block's (kblocks-1) wraps to the row's first dword, loaded once.
    const int cv_addr = (((lane & 15) << 2) | (lane >> 4)) << 2;  // transposed -> MFMA layout
    const int la_addr = ((lane + 16) & 63) << 2;                   // lane j+16g reads lane j+16(g+1)
    u32x4 aA[NS][4], aB[NS][4];
    if (APRE) load_a<NS, FRAG>(aA, p.act, aoff, kblocks - 1);
    const int ob_last = (kblocks - 1) * kCodeBlk + tc * 8;
    ChunkSet<NT> A0 = load_chunks<NT>(base0, roff, nt_stride, ob_last);
    ChunkSet<NT> A1 = (MODE == kModeGateUp) ? load_chunks<NT>(base1, roff, nt_stride, ob_last) : A0;
    uint32_t w0[NT], w1[NT];  // each row's first dword (every lane of its quad loads it)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      w0[nt] = *reinterpret_cast<const uint32_t*>(base0 + (roff + nt * nt_stride));
      w1[nt] = (MODE == kModeGateUp) ? *reinterpret_cast<const uint32_t*>(base1 + (roff + nt * nt_stride)) : w0[nt];
    }
    ChunkSet<NT> B0, B1;
    keep_apart(A0);
    if (MODE == kModeGateUp) keep_apart(A1);
    if (APRE) keep_apart<NS>(aA);
    uint32_t pA0[NT], pA1[NT], pB0[NT], pB1[NT];  // MFMA-layout d0 of the block decoded last
    // one block: decode c0/c1 (block kb = kblocks-1-s) against `acur`, with p0/p1 the previous
    // block's MFMA-layout d0 (FIRST: the row's first dword, still in transposed layout, in w0/w1);
    // block kb-1's codes go to n0/n1 and (APRE) its activations to `anext`; this block's d0 to q0/q1
    auto step = [&](auto first, int s, const ChunkSet<NT>& c0, const ChunkSet<NT>& c1, u32x4 (&acur)[NS][4],
                    const uint32_t (&p0)[NT], const uint32_t (&p1)[NT], ChunkSet<NT>& n0, ChunkSet<NT>& n1,
                    u32x4 (&anext)[NS][4], uint32_t (&q0)[NT], uint32_t (&q1)[NT]) {
      constexpr bool FIRST = decltype(first)::value;
      const int kb = kblocks - 1 - s;
      const int kn = kb > 0 ? kb - 1 : 0;
      const int ob = kn * kCodeBlk + tc * 8;
      if (MODE == kModeGateUp) {
        // fused pass: the next block's codes go out first, pinned before this block's first wait
        // (left to itself the scheduler sinks them below the waits for this block's data); its
        // activations may float, since pinning them too spills the fused kernels
        n0 = load_chunks<NT>(base0, roff, nt_stride, ob);
        n1 = load_chunks<NT>(base1, roff, nt_stride, ob);
        __builtin_amdgcn_sched_barrier(0);
        if (APRE) load_a<NS, FRAG>(anext, p.act, aoff, kn);
        else load_a<NS, FRAG>(acur, p.act, aoff, kb);
      } else {
        // single-matrix pass: activations, then codes, all pinned before this block's first wait
        if (APRE) load_a<NS, FRAG>(anext, p.act, aoff, kn);
        else load_a<NS, FRAG>(acur, p.act, aoff, kb);
        n0 = load_chunks<NT>(base0, roff, nt_stride, ob);
        __builtin_amdgcn_sched_barrier(0);
      }
      RunCodes m0[NT], m1[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t prev0 = FIRST ? (uint32_t)__builtin_amdgcn_ds_bpermute(cv_addr, (int)w0[nt]) : p0[nt];
        m0[nt] = chunk_to_mfma_layout(c0.c[nt], prev0, cv_addr, la_addr, g);
        q0[nt] = m0[nt].d0;
        if (MODE == kModeGateUp) {
          const uint32_t prev1 = FIRST ? (uint32_t)__builtin_amdgcn_ds_bpermute(cv_addr, (int)w1[nt]) : p1[nt];
          m1[nt] = chunk_to_mfma_layout(c1.c[nt], prev1, cv_addr, la_addr, g);
          q1[nt] = m1[nt].d0;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          u32x4 b0[2], b1[2];
          const RunCodes& x0 = m0[nt];
          lut.decode16(h ? x0.d1 : x0.d0, h ? x0.la : x0.d1, b0[0], b0[1]);
          if (MODE == kModeGateUp) {
            const RunCodes& x1 = m1[nt];
            lut.decode16(h ? x1.d1 : x1.d0, h ? x1.la : x1.d1, b1[0], b1[1]);
          }
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const int st = 2 * h + hs;
#pragma unroll
            for (int m = 0; m < NS; ++m) {
              acc0[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, acur[m][st]),
                                                                    __builtin_bit_cast(bf16x8, b0[hs]), acc0[m][nt], 0, 0, 0);
              if (MODE == kModeGateUp)
                acc1[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, acur[m][st]),
                                                                      __builtin_bit_cast(bf16x8, b1[hs]), acc1[m][nt], 0, 0, 0);
            }
          }
        }
      }
      // keep the next block's decode (which reads the codes just requested) after this block's work
      __builtin_amdgcn_sched_barrier(0);
    };
    using First = std::integral_constant<bool, true>;
    using Later = std::integral_constant<bool, false>;
    step(First{}, 0, A0, A1, aA, pA0, pA1, B0, B1, aB, pB0, pB1);
    int s = 1;
    for (; s + 1 < kblocks; s += 2) {
      step(Later{}, s, B0, B1, aB, pB0, pB1, A0, A1, aA, pA0, pA1);
      step(Later{}, s + 1, A0, A1, aA, pA0, pA1, B0, B1, aB, pB0, pB1);
    }
    if (s < kblocks) step(Later{}, s, B0, B1, aB, pB0, pB1, A0, A1, aA, pA0, pA1);
  }

  grouped_epilogue<MODE, NS, NT>(p, un, r0, acc0, acc1, pre);
}

// GEMV arm: NQ pairs x NT row blocks of 16 outputs share one decode; VALU bf16 dot products.
// GEMV arm body over the 128-input blocks [kb_lo, kb_hi) of a task (unit un, rows r0..): each
// lane accumulates its row's dot products with the NQ pairs over its quarter of each block
// into acc0 (gate or the single matrix) and acc1 (up).  A range holding the row's last block
// takes it first (its look-ahead wraps to the row start), then blocks kb_lo.. in order.
template <int MODE, int NQ, int NT, bool APRE, bool DEEP, class DEC>
__device__ inline void gemv_range(const ExpertParams& p, const DEC& lut, const Unit& un, int r0, int kb_lo,
                                  int kb_hi, float (&acc0)[NQ][NT], float (&acc1)[NQ][NT]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int row_bytes = p.cols >> 2;
  const int kblocks = p.cols / kKBlock;
  // matrix bases are wave-uniform; each lane's row is a 32-bit byte offset from them
  const size_t mat_bytes = (size_t)p.rows * row_bytes;
  const uint8_t* base0 = p.codes0 + (size_t)un.e * mat_bytes;
  const uint8_t* base1 = (MODE == kModeGateUp) ? p.codes1 + (size_t)un.e * mat_bytes : base0;
  // this lane's code chunk and row: transposed for a pipelined decoder (LUT rung, block-interleaved
  // codes), the MFMA layout otherwise
  const int tc = DEC::kPipelined ? code_chunk(lane) : g;
  const uint32_t roff = code_blk_row(r0 + (DEC::kPipelined ? code_row(lane) : j), row_bytes);
  const uint32_t nt_stride = 16u * (uint32_t)row_bytes;
  const bool wraps = kb_hi == kblocks;
  const int len = kb_hi - kb_lo;
  // the i-th block of the range's order
  auto block_of = [&](int i) { return wraps ? (i == 0 ? kblocks - 1 : kb_lo + i - 1) : kb_lo + i; };

  uint32_t xoff[NQ];  // every lane of group g reads the same 16 bytes of pair q
  act_rows<NQ>(p, un, 0, 1, g, xoff);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc0[q][nt] = acc1[q][nt] = 0.f;
  }

  if constexpr (!DEC::kPipelined && DEEP) {
    // DEEP (where the registers allow): with the block-interleaved storage each block's codes lie
    // in lines no earlier block read, and where a small launch leaves little work per block one
    // block does not cover the memory round trip.  So the look-ahead dwords (the chunk-3 lanes'
    // lie in the next block's lines) are loaded two blocks ahead, in two register sets (A for
    // even iterations, B for odd), and bring in the lines the next block's chunks, loaded one
    // block ahead, then read.  Past the range's end the loads re-read its first block (unused).
    u32x4 xn[NQ][4];
    if (APRE) load_a_block<NQ>(xn, p.act, xoff, block_of(0));
    auto blk = [&](int i) { return i < len ? block_of(i) : kb_lo; };
    ChunkSet<NT> n0 = load_chunks<NT>(base0, roff, nt_stride, blk(0) * kCodeBlk + tc * 8);
    ChunkSet<NT> n1 = (MODE == kModeGateUp) ? load_chunks<NT>(base1, roff, nt_stride, blk(0) * kCodeBlk + tc * 8) : n0;
    uint32_t lA0[NT], lA1[NT], lB0[NT], lB1[NT];
    load_las_blk<NT>(lA0, base0, roff, nt_stride, blk(0), tc, kblocks);
    load_las_blk<NT>(lB0, base0, roff, nt_stride, blk(1), tc, kblocks);
    if (MODE == kModeGateUp) {
      load_las_blk<NT>(lA1, base1, roff, nt_stride, blk(0), tc, kblocks);
      load_las_blk<NT>(lB1, base1, roff, nt_stride, blk(1), tc, kblocks);
    }
    auto step = [&](int i, uint32_t (&l0)[NT], uint32_t (&l1)[NT]) {
      const int kb = block_of(i);
      const int kn = blk(i + 1);
      u32x4 x[NQ][4];
      if (APRE) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
          for (int st = 0; st < 4; ++st) x[q][st] = xn[q][st];
        }
        load_a_block<NQ>(xn, p.act, xoff, kn);
      } else {
        load_a_block<NQ>(x, p.act, xoff, kb);
      }
      RunSet<NT> c0, c1;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        c0.c[nt] = RunCodes{n0.c[nt].d0, n0.c[nt].d1, l0[nt]};
        if (MODE == kModeGateUp) c1.c[nt] = RunCodes{n1.c[nt].d0, n1.c[nt].d1, l1[nt]};
      }
      n0 = load_chunks<NT>(base0, roff, nt_stride, kn * kCodeBlk + tc * 8);
      load_las_blk<NT>(l0, base0, roff, nt_stride, blk(i + 2), tc, kblocks);
      if (MODE == kModeGateUp) {
        n1 = load_chunks<NT>(base1, roff, nt_stride, kn * kCodeBlk + tc * 8);
        load_las_blk<NT>(l1, base1, roff, nt_stride, blk(i + 2), tc, kblocks);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          u32x4 b0[2], b1[2];
          const RunCodes& x0 = c0.c[nt];
          lut.decode16(h ? x0.d1 : x0.d0, h ? x0.la : x0.d1, b0[0], b0[1]);
          if (MODE == kModeGateUp) {
            const RunCodes& x1 = c1.c[nt];
            lut.decode16(h ? x1.d1 : x1.d0, h ? x1.la : x1.d1, b1[0], b1[1]);
          }
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              acc0[q][nt] = dot8(b0[hs], x[q][2 * h + hs], acc0[q][nt]);
              if (MODE == kModeGateUp) acc1[q][nt] = dot8(b1[hs], x[q][2 * h + hs], acc1[q][nt]);
            }
          }
        }
      }
    };
    for (int i = 0; i < len; i += 2) {
      step(i, lA0, lA1);
      if (i + 1 < len) step(i + 1, lB0, lB1);
    }
  } else if constexpr (!DEC::kPipelined) {
    u32x4 xn[NQ][4];
    if (APRE) load_a_block<NQ>(xn, p.act, xoff, block_of(0));
    RunSet<NT> n0 = load_runs_blk<NT>(base0, roff, nt_stride, block_of(0), tc, kblocks);
    RunSet<NT> n1 = (MODE == kModeGateUp) ? load_runs_blk<NT>(base1, roff, nt_stride, block_of(0), tc, kblocks) : n0;
    for (int i = 0; i < len; ++i) {
      const int kb = block_of(i);
      // the next block; after the last, the range's first in-row block again (unused)
      const int kn = i + 1 < len ? block_of(i + 1) : kb_lo;
      u32x4 x[NQ][4];
      if (APRE) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
          for (int st = 0; st < 4; ++st) x[q][st] = xn[q][st];
        }
        load_a_block<NQ>(xn, p.act, xoff, kn);
      } else {
        load_a_block<NQ>(x, p.act, xoff, kb);
      }
      const RunSet<NT> c0 = n0, c1 = n1;
      n0 = load_runs_blk<NT>(base0, roff, nt_stride, kn, tc, kblocks);
      if (MODE == kModeGateUp) n1 = load_runs_blk<NT>(base1, roff, nt_stride, kn, tc, kblocks);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          u32x4 b0[2], b1[2];
          const RunCodes& x0 = c0.c[nt];
          lut.decode16(h ? x0.d1 : x0.d0, h ? x0.la : x0.d1, b0[0], b0[1]);
          if (MODE == kModeGateUp) {
            const RunCodes& x1 = c1.c[nt];
            lut.decode16(h ? x1.d1 : x1.d0, h ? x1.la : x1.d1, b1[0], b1[1]);
          }
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              acc0[q][nt] = dot8(b0[hs], x[q][2 * h + hs], acc0[q][nt]);
              if (MODE == kModeGateUp) acc1[q][nt] = dot8(b1[hs], x[q][2 * h + hs], acc1[q][nt]);
            }
          }
        }
      }
    }
  } else {
    // ping-pong buffers, as in task_grouped: no register copy between blocks
    u32x4 xA[NQ][4], xB[NQ][4];
    if (APRE) load_a_block<NQ>(xA, p.act, xoff, block_of(0));
    RunSet<NT> A0, A1, B0, B1;
    A0 = load_runs_blk<NT>(base0, roff, nt_stride, block_of(0), tc, kblocks);
    A1 = (MODE == kModeGateUp) ? load_runs_blk<NT>(base1, roff, nt_stride, block_of(0), tc, kblocks) : A0;
    keep_apart(A0);
    if (MODE == kModeGateUp) keep_apart(A1);
    if (APRE) keep_apart<NQ>(xA);
    auto step = [&](int i, const RunSet<NT>& c0, const RunSet<NT>& c1, u32x4 (&x)[NQ][4], RunSet<NT>& n0,
                    RunSet<NT>& n1, u32x4 (&xnext)[NQ][4]) {
      const int kb = block_of(i);
      // the next block; after the last, the range's first in-row block again (unused)
      const int kn = i + 1 < len ? block_of(i + 1) : kb_lo;
      if (APRE) load_a_block<NQ>(xnext, p.act, xoff, kn);
      else load_a_block<NQ>(x, p.act, xoff, kb);
      n0 = load_runs_blk<NT>(base0, roff, nt_stride, kn, tc, kblocks);
      if (MODE == kModeGateUp) n1 = load_runs_blk<NT>(base1, roff, nt_stride, kn, tc, kblocks);
      // the next block's loads stay ahead of this block's first wait (see task_grouped)
      __builtin_amdgcn_sched_barrier(0);
      const RunSet<NT> m0 = to_mfma_layout(c0);
      const RunSet<NT> m1 = (MODE == kModeGateUp) ? to_mfma_layout(c1) : m0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          u32x4 b0[2], b1[2];
          const RunCodes& x0 = m0.c[nt];
          lut.decode16(h ? x0.d1 : x0.d0, h ? x0.la : x0.d1, b0[0], b0[1]);
          if (MODE == kModeGateUp) {
            const RunCodes& x1 = m1.c[nt];
            lut.decode16(h ? x1.d1 : x1.d0, h ? x1.la : x1.d1, b1[0], b1[1]);
          }
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              acc0[q][nt] = dot8(b0[hs], x[q][2 * h + hs], acc0[q][nt]);
              if (MODE == kModeGateUp) acc1[q][nt] = dot8(b1[hs], x[q][2 * h + hs], acc1[q][nt]);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // as in task_grouped
    };
    int i = 0;
    for (; i + 1 < len; i += 2) {
      step(i, A0, A1, xA, B0, B1, xB);
      step(i + 1, B0, B1, xB, A0, A1, xA);
    }
    if (i < len) step(i, A0, A1, xA, B0, B1, xB);
  }
}

// GEMV arm: sum the four lane groups' partial dot products of each row (lanes j, j+16, j+32,
// j+48) and store the NQ pairs' outputs.
template <int MODE, int NQ, int NT>
__device__ inline void gemv_epilogue(const ExpertParams& p, const Unit& un, int r0, const float (&acc0)[NQ][NT],
                                     const float (&acc1)[NQ][NT]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + 16 * nt + j;
    const float s0 = f16_to_f32(p.scale0[(size_t)un.e * p.rows + r]);
    const float s1 = (MODE == kModeGateUp) ? f16_to_f32(p.scale1[(size_t)un.e * p.rows + r]) : 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float a0 = acc0[q][nt];
      a0 += __shfl_xor(a0, 16, 64);
      a0 += __shfl_xor(a0, 32, 64);
      float a1 = 0.f;
      if (MODE == kModeGateUp) {
        a1 = acc1[q][nt];
        a1 += __shfl_xor(a1, 16, 64);
        a1 += __shfl_xor(a1, 32, 64);
      }
      if (q < un.len && (q & 3) == g)
        epilogue_store<MODE>(p, un, r, q, a0, a1, s0, s1, MODE == kModeSingle ? out_row(p, un.start + q) : -1);
    }
  }
}

// GEMV arm: the NQ pairs of a unit chunk against 16*NT rows of its expert (the per-pair dot
// products on the VALU, the decode in registers from the LDS LUT).
template <int MODE, int NQ, int NT, bool APRE, bool DEEP = false, class DEC = DecoderBitshift>
__device__ void task_gemv(const ExpertParams& p, const DEC& lut, const Unit& un, int r0) {
  float acc0[NQ][NT], acc1[NQ][NT];
  gemv_range<MODE, NQ, NT, APRE, DEEP>(p, lut, un, r0, 0, p.cols / kKBlock, acc0, acc1);
  gemv_epilogue<MODE, NQ, NT>(p, un, r0, acc0, acc1);
}

// GEMV arm with each task's inputs split over S waves of a workgroup (ExpertParams::ksplit),
// for launches with fewer tasks than the GPU has wave slots: wave s of a task's group decodes
// blocks [s K/S, (s+1) K/S) and leaves its partial sums in LDS; after a barrier the group's first
// wave adds the S partials in ascending s and stores the outputs.
template <int MODE, int NQ, int NT, bool APRE, bool DEEP, class DEC>
__device__ inline void gemv_part(const ExpertParams& p, const DEC& lut, const Unit& un, int r0, int kb_lo,
                                 int kb_hi, float* slot) {
  float acc0[NQ][NT], acc1[NQ][NT];
  gemv_range<MODE, NQ, NT, APRE, DEEP>(p, lut, un, r0, kb_lo, kb_hi, acc0, acc1);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      slot[((q * NT + nt) * 2 + 0) * 64 + lane] = acc0[q][nt];
      if (MODE == kModeGateUp) slot[((q * NT + nt) * 2 + 1) * 64 + lane] = acc1[q][nt];
    }
  }
}

template <int MODE, int NQ, int NT>
__device__ inline void gemv_finish(const ExpertParams& p, const Unit& un, int r0, const float* slots, int slot_floats,
                                   int S) {
  const int lane = threadIdx.x & 63;
  float acc0[NQ][NT], acc1[NQ][NT];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float a0 = 0.f, a1 = 0.f;
      for (int w = 0; w < S; ++w) {
        a0 += slots[w * slot_floats + ((q * NT + nt) * 2 + 0) * 64 + lane];
        if (MODE == kModeGateUp) a1 += slots[w * slot_floats + ((q * NT + nt) * 2 + 1) * 64 + lane];
      }
      acc0[q][nt] = a0;
      acc1[q][nt] = a1;
    }
  }
  gemv_epilogue<MODE, NQ, NT>(p, un, r0, acc0, acc1);
}

// A small batch's expert ids in workgroup memory (SmallRoute).
struct SmallRouteLds {
  int32_t idx[kSmallRouteMaxPairs];
};

// LDS the split-input GEMV path needs beside the LUT (and a small batch's routing): every wave's
// partial sums.
template <class CFG>
struct GemvSplit {
  static constexpr int kSlotFloats = CFG::kGPairs * CFG::kNT * 2 * 64;
  static constexpr int kFloats = CFG::kWaves * kSlotFloats;
  static constexpr bool kFits = kFloats * 4 <= 160 * 1024 - kLutEntries * 2 - (int)sizeof(SmallRouteLds);
};

// TokenCombine: the first wave adds the k x S partial sums of one token's 16 NT rows into the
// layer output (the sums as the split GEMV path and the combine kernel form them: ascending s, the
// lane groups' reduction, the row scale, then ascending j weighted by the router weights).
template <int NT>
__device__ inline void token_finish(const ExpertParams& p, int t, int r0, const float* part, int slot_floats,
                                    int S) {
  const TokenCombine& tc = p.tok;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + 16 * nt + (lane & 15);
    float acc = 0.f;
    for (int jj = 0; jj < tc.k; ++jj) {
      const int pair = t * tc.k + jj;
      const int e = __builtin_amdgcn_readfirstlane(tc.topk_idx[pair]);
      if (e < 0 || e >= p.num_experts) continue;
      float a0 = 0.f;
      for (int w = 0; w < S; ++w) a0 += part[(jj * S + w) * slot_floats + nt * 2 * 64 + lane];
      a0 += __shfl_xor(a0, 16, 64);
      a0 += __shfl_xor(a0, 32, 64);
      const float y = a0 * f16_to_f32(p.scale0[(size_t)e * p.rows + r]);
      acc = fmaf(tc.topk_w[pair], y, acc);
    }
    if (lane < 16) {
      const size_t o = (size_t)t * p.rows + r;
      if (tc.out_bf16) reinterpret_cast<uint16_t*>(tc.out)[o] = (uint16_t)f32_to_bf16_bits(acc);
      else reinterpret_cast<float*>(tc.out)[o] = acc;
    }
  }
}

// TokenCombine's task loop: a workgroup of k x S waves per token task (waves past k S idle).
template <class CFG, class DEC>
__device__ inline void gemv_token_tasks(const ExpertParams& p, const DEC& lut, float* part) {
  constexpr int NT = CFG::kNT;
  constexpr bool AP = CFG::kAPre;
  constexpr int kSlot = GemvSplit<CFG>::kSlotFloats;
  const TokenCombine& tc = p.tok;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = p.ksplit > 1 ? p.ksplit : 1;
  const int j = wave / S, sidx = wave % S;
  const int kper = p.cols / kKBlock / S;
  const int lo = sidx * kper, hi = lo + kper;
  const int nblocks = p.rows / CFG::kRows;
  const long total = (long)tc.n * nblocks;
  float* mine = part + wave * kSlot;
  for (long task = blockIdx.x; task < total; task += gridDim.x) {
    const int t = (int)(task / nblocks);
    const int r0 = (int)(task - (long)t * nblocks) * CFG::kRows;
    if (j < tc.k) {
      const int pair = t * tc.k + j;
      const int e = __builtin_amdgcn_readfirstlane(tc.topk_idx[pair]);
      if (e >= 0 && e < p.num_experts) {
        const Unit un{e, __builtin_amdgcn_readfirstlane(tc.pair_pos[pair]), 1, -1};
        gemv_part<kModeSingle, 1, NT, AP, CFG::kDeepGemvDown>(p, lut, un, r0, lo, hi, mine);
      }
    }
    __syncthreads();
    if (wave == 0) token_finish<NT>(p, t, r0, part, kSlot, S);
    __syncthreads();
  }
}

// SmallRoute, step 1: the workgroup's waves route the batch's tokens (token t by wave t modulo
// the waves) into workgroup memory; workgroup 0 also stores the expert ids and router weights.
__device__ inline void small_route_tokens(const ExpertParams& p, SmallRouteLds& rs) {
  const SmallRoute& r = p.route;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = (int)(blockDim.x >> 6);
  const bool first = blockIdx.x == 0;
  for (int t = wave; t < r.n; t += nw) {
    int32_t* idx2 = first ? r.topk_idx : nullptr;
    float* w = first ? r.topk_w : nullptr;
    if (p.num_experts <= 256) route_token<4>(r.logits, r.n_part, r.n, p.num_experts, r.top_k, t, rs.idx, idx2, w);
    else route_token<16>(r.logits, r.n_part, r.n, p.num_experts, r.top_k, t, rs.idx, idx2, w);
  }
}

// SmallRoute, step 2, by one wave once the ids are in workgroup memory: the stable counting sort
// of the P <= 64 pairs by expert (lane p holds pair p) and the runs that cut each expert's bin
// into the two passes' units, stored as the binning kernel stores them (out-of-range ids are left
// out).  A pair's binned position is the number of valid pairs of lower experts plus the number
// of its expert's pairs before it; a unit starts at every unit_pairs-th pair of a bin, and a
// unit's index is the number of unit starts at lower positions.  Every workgroup stores what its
// own tasks read back after a workgroup barrier (the binned order and the gate/up units: the same
// values from every workgroup); workgroup 0 also stores the down pass's units.
__device__ inline void small_bin(const ExpertParams& p, const SmallRouteLds& rs) {
  const SmallRoute& r = p.route;
  const int lane = threadIdx.x & 63;
  const int E = p.num_experts, P = r.n * r.top_k;
  int e = lane < P ? rs.idx[lane] : E;
  const bool valid = lane < P && e >= 0 && e < E;
  if (!valid) e = E;
  int below = 0, same = 0, rank = 0;
  for (int q = 0; q < P; ++q) {
    const int eq = __builtin_amdgcn_readlane(e, q);
    below += eq < e;
    same += eq == e;
    rank += (eq == e) & (q < lane);
  }
  const int pos = below + rank;
  const int U0 = r.unit_pairs[0], U1 = r.unit_pairs[1];
  const bool s0 = valid && rank % U0 == 0, s1 = valid && rank % U1 == 0;
  const uint64_t m0 = __ballot(s0), m1 = __ballot(s1);
  int u0 = 0, u1 = 0;
  for (int q = 0; q < P; ++q) {
    const bool lower = __builtin_amdgcn_readlane(pos, q) < pos;
    u0 += (int)((m0 >> q) & 1u) & lower;
    u1 += (int)((m1 >> q) & 1u) & lower;
  }
  if (valid) r.sorted_pair[pos] = lane;
  if (s0) {
    r.units[0][3 * u0 + 0] = e;
    r.units[0][3 * u0 + 1] = pos;
    r.units[0][3 * u0 + 2] = min(U0, same - rank);
  }
  if (lane == 0) *r.n_units[0] = __popcll(m0);
  if (blockIdx.x != 0) return;
  if (r.pair_pos && lane < P) r.pair_pos[lane] = valid ? pos : -1;
  if (s1) {
    r.units[1][3 * u1 + 0] = e;
    r.units[1][3 * u1 + 1] = pos;
    r.units[1][3 * u1 + 2] = min(U1, same - rank);
  }
  if (lane == 0) *r.n_units[1] = __popcll(m1);
}

// Kernel configurations (the plan's `variant`): waves per workgroup, 16-row output blocks
// per task (NT), pairs per decode on the grouped arm (in 16-pair MFMA row blocks, NSUB) and
// on the GEMV arm.  Fewer waves leave each wave more registers; more rows per task feed each
// activation fragment to more MFMAs; more pairs per decode mean fewer decodes.
template <int WAVES, int NT, int NSUB, int GPAIRS>
struct ExpertCfg {
  static constexpr int kWaves = WAVES, kNT = NT, kNSub = NSUB, kGPairs = GPAIRS;
  static constexpr int kRows = 16 * NT;
  // Activation double-buffering where the register budget allows it: 512 VGPRs per SIMD lane
  // shared by WAVES/4 waves (168 at 12 waves, where the 4-block task, or three 16-pair blocks
  // per decode, would spill).
  static constexpr bool kAPre = WAVES <= 8 || (NT <= 2 && NSUB <= 2);
  // GEMV arm: look-ahead dwords loaded two blocks ahead (gemv_range) where the registers allow it:
  // the fused pass at up to 12 waves and 16 rows, the single-matrix pass up to 12 waves and 8
  // row-pair products per lane (larger tasks spill).
  static constexpr bool kDeepGemvGateUp = WAVES <= 12 && NT == 1;
  static constexpr bool kDeepGemvDown = NT == 1 || (WAVES <= 12 && NT * GPAIRS <= 8);
  // The fused grouped task of 64 rows x three 16-pair blocks would spill heavily at 12 waves;
  // that configuration serves the down pass only (the plan runs the fused pass as 32-row tasks).
  static constexpr bool kGroupedFused = !(NT == 4 && NSUB >= 3);
};
using Cfg1 = ExpertCfg<16, 1, 2, 2>;
using Cfg2 = ExpertCfg<8, 1, 4, 4>;
using Cfg3 = ExpertCfg<16, 2, 2, 2>;
using Cfg4 = ExpertCfg<8, 2, 4, 4>;
using Cfg5 = ExpertCfg<8, 4, 2, 2>;
using Cfg6 = ExpertCfg<12, 2, 2, 2>;
using Cfg7 = ExpertCfg<12, 4, 2, 2>;
// One decode per 16-pair m-tile (no sharing across m-tiles): the pages' grouped-kernel
// schedule, kept to measure what sharing a decode across m-tiles is worth.
using Cfg8 = ExpertCfg<16, 1, 1, 1>;
// 12 waves of 32-row tasks sharing a decode across three 16-pair blocks (48 pairs).
using Cfg9 = ExpertCfg<12, 2, 3, 3>;
// 12 waves of 64-row tasks sharing a decode across three 16-pair blocks (48 pairs): a down-pass
// shape (see kGroupedFused).
using Cfg10 = ExpertCfg<12, 4, 3, 3>;
// 12 waves of 16-row tasks sharing a decode across three 16-pair blocks (48 pairs): the decode
// sharing of variant 9 with half the code rows in flight per task, so that the code lines a task
// reads over four consecutive blocks (each 128-byte line holds four blocks of a row) stay in the
// XCD's L2 between their uses.
using Cfg11 = ExpertCfg<12, 1, 3, 3>;

// The grouped body specialised for the chunk's exact number of 16-pair row blocks.
template <int MODE, class CFG, bool FRAG, class DEC>
__device__ inline void grouped_blocks(const ExpertParams& p, const DEC& lut, const Unit& part, int r0) {
  constexpr int NT = CFG::kNT;
  constexpr bool AP = CFG::kAPre;
  switch ((part.len + 15) >> 4) {
    case 1: task_grouped<MODE, 1, NT, AP, FRAG>(p, lut, part, r0); break;
    case 2: if (CFG::kNSub >= 2) task_grouped<MODE, (CFG::kNSub >= 2 ? 2 : 1), NT, AP, FRAG>(p, lut, part, r0); break;
    case 3: if (CFG::kNSub >= 3) task_grouped<MODE, (CFG::kNSub >= 3 ? 3 : 1), NT, AP, FRAG>(p, lut, part, r0); break;
    default: if (CFG::kNSub >= 4) task_grouped<MODE, (CFG::kNSub >= 4 ? 4 : 1), NT, AP, FRAG>(p, lut, part, r0); break;
  }
}

// A unit may hold more pairs than one decode serves; it is then processed in chunks, each
// chunk decoding the rows again.  Each chunk runs the body specialised for its exact number
// of 16-pair row blocks (grouped) or pairs (GEMV), chosen by a wave-uniform switch.
template <int MODE, int ARM, class CFG, bool FRAG, class DEC>
__device__ inline void run_task(const ExpertParams& p, const DEC& lut, const Unit& un, int r0) {
  constexpr int NT = CFG::kNT;
  constexpr bool AP = CFG::kAPre;
  constexpr int kChunk = (ARM == kArmGemv) ? CFG::kGPairs : CFG::kNSub * 16;
  constexpr bool DEEP = MODE == kModeSingle ? CFG::kDeepGemvDown : CFG::kDeepGemvGateUp;
  static_assert(CFG::kNSub >= 1 && CFG::kNSub <= 4 && CFG::kGPairs >= 1 && CFG::kGPairs <= 4, "config");
  for (int c0 = 0; c0 < un.len; c0 += kChunk) {
    const Unit part{un.e, un.start + c0, min(kChunk, un.len - c0), un.pad >= 0 ? un.pad + c0 : -1};
    if (ARM == kArmDense) {
      switch ((part.len + 15) >> 4) {
        case 1: task_dense<MODE, 1, NT>(p, part, r0); break;
        case 2: if (CFG::kNSub >= 2) task_dense<MODE, (CFG::kNSub >= 2 ? 2 : 1), NT>(p, part, r0); break;
        case 3: if (CFG::kNSub >= 3) task_dense<MODE, (CFG::kNSub >= 3 ? 3 : 1), NT>(p, part, r0); break;
        default: if (CFG::kNSub >= 4) task_dense<MODE, (CFG::kNSub >= 4 ? 4 : 1), NT>(p, part, r0); break;
      }
    } else if (ARM == kArmGrouped) {
      grouped_blocks<MODE, CFG, FRAG>(p, lut, part, r0);
    } else {
      switch (part.len) {
        case 1: task_gemv<MODE, 1, NT, AP, DEEP>(p, lut, part, r0); break;
        case 2: if (CFG::kGPairs >= 2) task_gemv<MODE, (CFG::kGPairs >= 2 ? 2 : 1), NT, AP, DEEP>(p, lut, part, r0); break;
        case 3: if (CFG::kGPairs >= 3) task_gemv<MODE, (CFG::kGPairs >= 3 ? 3 : 1), NT, AP, DEEP>(p, lut, part, r0); break;
        default: if (CFG::kGPairs >= 4) task_gemv<MODE, (CFG::kGPairs >= 4 ? 4 : 1), NT, AP, DEEP>(p, lut, part, r0); break;
      }
    }
  }
}

// The GEMV arm's task loop with split inputs: a workgroup of tpw x S waves takes tpw tasks per
// round, S waves each (every wave runs the same rounds, so the barriers line up).
template <int MODE, class CFG, class DEC>
__device__ inline void gemv_split_tasks(const ExpertParams& p, const DEC& lut, float* part) {
  constexpr int NT = CFG::kNT;
  constexpr bool AP = CFG::kAPre;
  constexpr int kSlot = GemvSplit<CFG>::kSlotFloats;
  constexpr bool DEEP = MODE == kModeSingle ? CFG::kDeepGemvDown : CFG::kDeepGemvGateUp;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = p.ksplit, tpw = (int)(blockDim.x >> 6) / S;
  const int q = wave / S, sidx = wave % S;
  const int kper = p.cols / kKBlock / S;
  const int n_units = p.n_units_dev ? __builtin_amdgcn_readfirstlane(*p.n_units_dev) : p.n_units_host;
  const int nblocks = p.rows / CFG::kRows;
  const long total = (long)n_units * nblocks;
  float* mine = part + wave * kSlot;
  for (long base = (long)blockIdx.x * tpw; base < total; base += (long)gridDim.x * tpw) {
    const long t = base + q;
    Unit un{};
    const bool ok = t < total && read_unit(p, (int)(t / nblocks), un);
    const int r0 = (int)(t % nblocks) * CFG::kRows;
    const bool one = ok && un.len <= CFG::kGPairs;  // a single chunk (the layer's own units)
    const int lo = sidx * kper, hi = lo + kper;
    if (one) {
      switch (un.len) {
        case 1: gemv_part<MODE, 1, NT, AP, DEEP>(p, lut, un, r0, lo, hi, mine); break;
        case 2: if (CFG::kGPairs >= 2) gemv_part<MODE, (CFG::kGPairs >= 2 ? 2 : 1), NT, AP, DEEP>(p, lut, un, r0, lo, hi, mine); break;
        case 3: if (CFG::kGPairs >= 3) gemv_part<MODE, (CFG::kGPairs >= 3 ? 3 : 1), NT, AP, DEEP>(p, lut, un, r0, lo, hi, mine); break;
        default: if (CFG::kGPairs >= 4) gemv_part<MODE, (CFG::kGPairs >= 4 ? 4 : 1), NT, AP, DEEP>(p, lut, un, r0, lo, hi, mine); break;
      }
    }
    __syncthreads();
    if (ok && sidx == 0) {
      const float* slots = part + (q * S) * kSlot;
      if (one) {
        switch (un.len) {
          case 1: gemv_finish<MODE, 1, NT>(p, un, r0, slots, kSlot, S); break;
          case 2: if (CFG::kGPairs >= 2) gemv_finish<MODE, (CFG::kGPairs >= 2 ? 2 : 1), NT>(p, un, r0, slots, kSlot, S); break;
          case 3: if (CFG::kGPairs >= 3) gemv_finish<MODE, (CFG::kGPairs >= 3 ? 3 : 1), NT>(p, un, r0, slots, kSlot, S); break;
          default: if (CFG::kGPairs >= 4) gemv_finish<MODE, (CFG::kGPairs >= 4 ? 4 : 1), NT>(p, un, r0, slots, kSlot, S); break;
        }
      } else {
        run_task<MODE, kArmGemv, CFG, false>(p, lut, un, r0);  // a longer unit: its group's first wave alone
      }
    }
    __syncthreads();
  }
}

// SPREAD: the launch may run fewer waves per workgroup than the configuration's (a small
// batch spread over more CUs).
template <int MODE, int ARM, class CFG, bool FRAG, bool SPREAD, class DEC>
__device__ inline void expert_tasks(const ExpertParams& p, const DEC& lut_s) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = p.n_units_dev ? __builtin_amdgcn_readfirstlane(*p.n_units_dev) : p.n_units_host;
  const int nblocks = p.rows / CFG::kRows;
  const long total = (long)n_units * nblocks;
  // Task order.  Workgroup b runs on XCD b % n_xcd (round-robin dispatch).  Each XCD owns a
  // contiguous share of the tasks in proportion to its workgroups, and its waves take that
  // share's tasks in turn across its CUs, so an XCD works on a few units at a time: their
  // activation rows stay in its L2, and a CU's waves (row blocks of the same unit) share them
  // in L1.  Every unit is one decode, so equal task counts are equal work; share boundaries are
  // rounded to whole rounds of the XCD's CUs when those divide a unit's row blocks, so every CU
  // then takes the same row blocks of the same units.
  const int nx = p.n_xcd;
  const int G = gridDim.x;
  const int xcd = blockIdx.x % nx, cu = blockIdx.x / nx;
  const int cus = G / nx + (xcd < G % nx ? 1 : 0);
  const int before = xcd * (G / nx) + min(xcd, G % nx);
  long lo = total * before / G;
  long hi = total * (before + cus) / G;
  const long Q = G / nx;
  if (Q > 1 && nblocks % Q == 0) {
    lo = (lo + Q / 2) / Q * Q;
    hi = (hi + Q / 2) / Q * Q;
  }
  const long nslots = (long)(SPREAD ? (int)(blockDim.x >> 6) : CFG::kWaves) * cus;
  for (long task = lo + (long)wave * cus + cu; task < hi; task += nslots) {
    const int u = (int)(task / nblocks);
    const int nb = (int)(task - (long)u * nblocks);
    Unit un;
    if (!read_unit(p, u, un)) continue;
    run_task<MODE, ARM, CFG, FRAG>(p, lut_s, un, nb * CFG::kRows);
  }
}

// A pass's tasks once the decoder's table is in LDS.
template <int MODE, int ARM, class CFG, bool FRAG, bool SPREAD, class DEC>
__device__ inline void expert_pass(const ExpertParams& p, const DEC& dec) {
  if constexpr (ARM == kArmGemv && GemvSplit<CFG>::kFits && (SPREAD || MODE == kModeSingle)) {
    __shared__ float part[GemvSplit<CFG>::kFloats];
    if constexpr (MODE == kModeSingle) {
      if (p.tok.out) {
        gemv_token_tasks<CFG>(p, dec, part);
        return;
      }
    }
    if (SPREAD && p.ksplit > 1) {
      gemv_split_tasks<MODE, CFG>(p, dec, part);
      return;
    }
  }
  expert_tasks<MODE, ARM, CFG, FRAG, SPREAD>(p, dec);
}

// The fill of the decoder's table (ending in a workgroup barrier), then the pass.  The GEMV
// arm's fused pass may first route and bin a small batch itself (SmallRoute): the routing is
// issued before the fill and the binning follows it.
template <int MODE, int ARM, class CFG, bool FRAG, bool SPREAD, class FILL, class DEC>
__device__ inline void fill_and_run(const ExpertParams& p, const FILL& fill, const DEC& dec) {
  if constexpr (MODE == kModeGateUp && ARM == kArmGemv) {
    __shared__ SmallRouteLds rs;
    const bool route = p.route.logits != nullptr;
    if (route) small_route_tokens(p, rs);
    fill();
    if (route) {
      if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0) small_bin(p, rs);
      __syncthreads();
    }
    expert_pass<MODE, ARM, CFG, FRAG, SPREAD>(p, dec);
  } else {
    fill();
    expert_pass<MODE, ARM, CFG, FRAG, SPREAD>(p, dec);
  }
}

// FRAG: the grouped arm's activations are in fragment order (ExpertParams::act_frag).
// SPREAD (GEMV arm): the launch may run fewer waves per workgroup than CFG's.
// RUNG: the decode (kRungBitshift: the 128 KiB LUT in LDS; kRungLut: the 64 KiB replicated codebook).
template <int MODE, int ARM, class CFG, bool FRAG = false, bool SPREAD = false, int RUNG = kRungBitshift>
__global__ __launch_bounds__(CFG::kWaves * 64, 1) void expert_kernel(ExpertParams p) {
  if constexpr (ARM == kArmDense) {
    expert_tasks<MODE, ARM, CFG, false, false>(p, DecoderBitshift{nullptr});
  } else if constexpr (RUNG == kRungLut) {
    __shared__ __attribute__((aligned(16))) uint32_t cb_s[kCodebookEntries * kCodebookCopies];
    const DecoderLut dec{reinterpret_cast<const char*>(cb_s), (uint32_t)(threadIdx.x & 31) * 4u};
    fill_and_run<MODE, ARM, CFG, FRAG, SPREAD>(p, [&] { fill_codebook(cb_s, p.lut); }, dec);
  } else {
    __shared__ __attribute__((aligned(16))) uint16_t lut_s[kLutEntries];
    const DecoderBitshift dec{lut_s};
    fill_and_run<MODE, ARM, CFG, FRAG, SPREAD>(p, [&] {
      if constexpr (SPREAD) fill_lut_any(lut_s, p.lut);
      else fill_lut<CFG::kWaves * 64>(lut_s, p.lut);
    }, dec);
  }
}

// Dequantize-materialise: one wave task decodes 16 rows x all inputs of one matrix and stores
// bf16(LUT[state]), in row-major order or in the fragment order of the dequantize arm's MFMA
// pass (every store 1 KiB contiguous per wave), there as non-temporal stores (written once, read
// once by a later launch).
template <int RUNG>
__global__ __launch_bounds__(kDequantWaves * 64, 1) void dequant_kernel(DequantParams q) {
  __shared__ __attribute__((aligned(16))) uint16_t lut_s[RUNG == kRungLut ? 2 * kCodebookEntries * kCodebookCopies
                                                                          : kLutEntries];
  if constexpr (RUNG == kRungLut) fill_codebook(reinterpret_cast<uint32_t*>(lut_s), q.lut);
  else fill_lut<kDequantWaves * 64>(lut_s, q.lut);
  typedef typename std::conditional<RUNG == kRungLut, DecoderLut, DecoderBitshift>::type Dec;
  Dec dec{};
  if constexpr (RUNG == kRungLut) dec = DecoderLut{reinterpret_cast<const char*>(lut_s), (uint32_t)(threadIdx.x & 31) * 4u};
  else dec = DecoderBitshift{lut_s};
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_bytes = q.cols >> 2;
  const int kblocks = q.cols / kKBlock;
  const int nblocks = q.rows / 16;
  const int e_first = q.expert >= 0 ? q.expert : 0;
  // with counts, the tasks cover the woken experts only (slot s = the s-th woken expert), so that
  // every wave gets the same share of them
  const bool by_slot = q.expert < 0 && q.counts;
  const long n_exp = q.expert >= 0 ? 1 : (by_slot ? woken_count(q.counts, q.num_experts) : q.num_experts);
  // a task: one matrix's 16-row block (gate and up are separate tasks)
  const int nmat = q.codes1 ? 2 : 1;
  const long total = n_exp * nmat * nblocks;
  const size_t mat_bytes = (size_t)q.rows * row_bytes;
  for (long task = (long)blockIdx.x * kDequantWaves + wave; task < total; task += (long)gridDim.x * kDequantWaves) {
    const int s = (int)(task / ((long)nmat * nblocks));
    const int m = (int)((task / nblocks) % nmat);
    const int e = by_slot ? nth_woken(q.counts, q.num_experts, s) : e_first + s;
    const int rb = (int)(task % nblocks);
    const int r0 = rb * 16;
    if (e < 0) continue;  // counts changed under the launch: not reached
    const size_t slot = by_slot ? (size_t)s : (q.counts ? (size_t)dense_slot(q.counts, e) : (size_t)e);
    const uint8_t* base = (m ? q.codes1 : q.codes0) + (size_t)e * mat_bytes;
    uint16_t* out = (m ? q.out1 : q.out0) + slot * (size_t)q.out_expert_stride;
    // this lane's code chunk and row: transposed for a pipelined decoder, the MFMA layout otherwise
    const int tc = Dec::kPipelined ? code_chunk(lane) : g;
    const uint32_t roff = code_blk_row(r0 + (Dec::kPipelined ? code_row(lane) : j), row_bytes);
    if constexpr (!Dec::kPipelined) {
      auto rows = [&](auto frag) {
        constexpr bool FRAG = decltype(frag)::value;
        auto store_block = [&](const RunCodes& c, int kb) {
          u32x4 w[4];
          dec.decode16(c.d0, c.d1, w[0], w[1]);
          dec.decode16(c.d1, c.la, w[2], w[3]);
          if constexpr (FRAG) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
              __builtin_nontemporal_store(w[st], reinterpret_cast<u32x4*>(out + dense_fragment_offset(rb, kb, st, lane, kblocks)));
          } else {
            uint16_t* row = out + (size_t)(r0 + j) * q.cols + kb * kKBlock + 32 * g;
#pragma unroll
            for (int st = 0; st < 4; ++st) *reinterpret_cast<u32x4*>(row + 8 * st) = w[st];
          }
        };
        constexpr int B = kDqBatch;
        if (kblocks % (4 * B) != 0) {
          RunCodes nx = load_run_blk(base, roff, kblocks - 1, tc, kblocks);
          for (int i = 0; i < kblocks; ++i) {
            const RunCodes rc = nx;
            if (i + 1 < kblocks) nx = load_run_blk(base, roff, i, tc, kblocks);
            store_block(rc, block_at(i, kblocks));
          }
          return;
        }
        // One counter covers loads and stores, so a wait for codes also waits for every store
        // issued before their load.  Batches of B blocks in two register sets: the next
        // batch's codes are requested before this batch's stores, so a store is waited for a
        // batch later, not on the next block.  Four batches per iteration: at the loop head
        // the compiler's wait covers the previous batch's stores too.  (The last batch's loads
        // re-read the row's first blocks, unused.)
        auto load_batch = [&](RunCodes (&c)[B], int i0) {
#pragma unroll
          for (int b = 0; b < B; ++b)
            c[b] = load_run_blk(base, roff, block_at(i0 + b < kblocks ? i0 + b : 0, kblocks), tc, kblocks);
        };
        RunCodes cA[B], cB[B];
        load_batch(cA, 0);
        for (int i = 0; i < kblocks; i += 4 * B) {
#pragma unroll
          for (int h = 0; h < 4; h += 2) {
            load_batch(cB, i + (h + 1) * B);
#pragma unroll
            for (int b = 0; b < B; ++b) store_block(cA[b], block_at(i + h * B + b, kblocks));
            load_batch(cA, i + (h + 2) * B);
#pragma unroll
            for (int b = 0; b < B; ++b) store_block(cB[b], block_at(i + (h + 1) * B + b, kblocks));
          }
        }
      };
      if (q.fragment_order) rows(std::true_type{});
      else rows(std::false_type{});
      continue;
    }
    RunCodes cA = load_run_blk(base, roff, kblocks - 1, tc, kblocks), cB{};
    keep_apart(cA);
    auto step = [&](int i, const RunCodes& rc, RunCodes& nx) {
      const int kb = block_at(i, kblocks);
      if (i + 1 < kblocks) nx = load_run_blk(base, roff, i, tc, kblocks);
      const RunCodes mc = to_mfma_layout(rc);
      u32x4 w[4];
      dec.decode16(mc.d0, mc.d1, w[0], w[1]);
      dec.decode16(mc.d1, mc.la, w[2], w[3]);
      if (q.fragment_order) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
          __builtin_nontemporal_store(w[st], reinterpret_cast<u32x4*>(out + dense_fragment_offset(rb, kb, st, lane, kblocks)));
      } else {
        uint16_t* row = out + (size_t)(r0 + j) * q.cols + kb * kKBlock + 32 * g;
#pragma unroll
        for (int st = 0; st < 4; ++st) *reinterpret_cast<u32x4*>(row + 8 * st) = w[st];
      }
      __builtin_amdgcn_sched_barrier(0);  // as in task_grouped
    };
    int i = 0;
    for (; i + 1 < kblocks; i += 2) {
      step(i, cA, cB);
      step(i + 1, cB, cA);
    }
    if (i < kblocks) step(i, cA, cB);
  }
}

}  // namespace

// The dequantize arm runs one configuration (variant 3's shape: 16 waves, 32-row tasks, up to
// 32 pairs per pass over the weights).
using CfgDense = ExpertCfg<16, 2, 2, 2>;

template <class CFG, int RUNG>
static hipError_t launch_cfg(int mode, int arm, const ExpertParams& p, int grid, int waves, hipStream_t stream) {
  // only the GEMV arm is built to run with fewer waves than its configuration's
  const int full = arm == kArmDense ? CfgDense::kWaves : CFG::kWaves;
  if (grid < 1 || waves < 1 || waves > full || (waves < full && arm != kArmGemv)) return hipErrorInvalidValue;
  const dim3 g(grid), b(waves * 64);
  const bool spread = waves < full;
  if (arm == kArmDense) {
    if constexpr (RUNG != kRungBitshift) return hipErrorInvalidValue;  // rung-independent: launched once
    const dim3 bd(waves * 64);
    if (mode == kModeGateUp)
      hipLaunchKernelGGL((expert_kernel<kModeGateUp, kArmDense, CfgDense>), g, bd, 0, stream, p);
    else
      hipLaunchKernelGGL((expert_kernel<kModeSingle, kArmDense, CfgDense>), g, bd, 0, stream, p);
  } else if (mode == kModeGateUp && arm == kArmGrouped) {
    if constexpr (CFG::kGroupedFused) {
      if (p.act_frag && p.unit_pad)
        hipLaunchKernelGGL((expert_kernel<kModeGateUp, kArmGrouped, CFG, true, false, RUNG>), g, b, 0, stream, p);
      else
        hipLaunchKernelGGL((expert_kernel<kModeGateUp, kArmGrouped, CFG, false, false, RUNG>), g, b, 0, stream, p);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (mode == kModeGateUp) {
    if (spread)
      hipLaunchKernelGGL((expert_kernel<kModeGateUp, kArmGemv, CFG, false, true, RUNG>), g, b, 0, stream, p);
    else
      hipLaunchKernelGGL((expert_kernel<kModeGateUp, kArmGemv, CFG, false, false, RUNG>), g, b, 0, stream, p);
  } else if (arm == kArmGrouped) {
    if (p.act_frag && p.unit_pad)
      hipLaunchKernelGGL((expert_kernel<kModeSingle, kArmGrouped, CFG, true, false, RUNG>), g, b, 0, stream, p);
    else
      hipLaunchKernelGGL((expert_kernel<kModeSingle, kArmGrouped, CFG, false, false, RUNG>), g, b, 0, stream, p);
  } else if (spread) {
    hipLaunchKernelGGL((expert_kernel<kModeSingle, kArmGemv, CFG, false, true, RUNG>), g, b, 0, stream, p);
  } else {
    hipLaunchKernelGGL((expert_kernel<kModeSingle, kArmGemv, CFG, false, false, RUNG>), g, b, 0, stream, p);
  }
  return hipGetLastError();
}


// Every kernel configuration of one rung.
template <int RUNG>
static hipError_t launch_expert_rung(int mode, int arm, int variant, const ExpertParams& p, int grid, int waves,
                                     hipStream_t stream) {
  switch (variant) {
    case 1: return launch_cfg<Cfg1, RUNG>(mode, arm, p, grid, waves, stream);
    case 2: return launch_cfg<Cfg2, RUNG>(mode, arm, p, grid, waves, stream);
    case 3: return launch_cfg<Cfg3, RUNG>(mode, arm, p, grid, waves, stream);
    case 4: return launch_cfg<Cfg4, RUNG>(mode, arm, p, grid, waves, stream);
    case 5: return launch_cfg<Cfg5, RUNG>(mode, arm, p, grid, waves, stream);
    case 6: return launch_cfg<Cfg6, RUNG>(mode, arm, p, grid, waves, stream);
    case 7: return launch_cfg<Cfg7, RUNG>(mode, arm, p, grid, waves, stream);
    case 8: return launch_cfg<Cfg8, RUNG>(mode, arm, p, grid, waves, stream);
    case 9: return launch_cfg<Cfg9, RUNG>(mode, arm, p, grid, waves, stream);
    case 10: return launch_cfg<Cfg10, RUNG>(mode, arm, p, grid, waves, stream);
    case 11: return launch_cfg<Cfg11, RUNG>(mode, arm, p, grid, waves, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int RUNG>
static hipError_t launch_dequant_rung(const DequantParams& q, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(dequant_kernel<RUNG>, dim3(grid), dim3(kDequantWaves * 64), 0, stream, q);
  return hipGetLastError();
}

}  // namespace qtip
