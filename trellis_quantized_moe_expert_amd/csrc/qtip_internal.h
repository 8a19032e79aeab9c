// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace qtip {

constexpr int kLutEntries = 65536;     // 16-bit trellis state -> one LUT entry (bitshift rung)
// The two 2-bit rungs: the bitshift rung (one weight per 16-bit window, a 65536-entry LUT) and the
// LUT rung (one 2-D codebook vector per 9-bit pair state, a 512 x 2 codebook).
enum Rung { kRungBitshift = 0, kRungLut = 1 };
constexpr int kLutRungBits = 9;                      // pair-state bits of the LUT rung
constexpr int kCodebookEntries = 1 << kLutRungBits;  // 512 two-dimensional entries
constexpr int kCodebookCopies = 32;                  // one copy per LDS bank (see DecoderLut)
// The LUT fills 128 KiB of LDS, so one expert workgroup per CU is resident; the kernel
// variant fixes its size (8, 12 or 16 wave64; a small GEMV launch may run fewer).
// Variants 1..11 are fixed kernel configurations (see variant_info); 0 lets the plan choose.
enum ExpertVariant { kVariantDefault = 0, kVariantCount = 12 };
constexpr int kExpertWaves = 16;       // waves of the binning workgroup
constexpr int kBinCached = 8;          // groups of 64 expert ids a binning wave keeps in registers
constexpr int kKBlock = 128;           // inputs per K block: 4 lane groups x 32-symbol runs
constexpr int kUnitMaxPairs = 64;      // most pairs one decode serves (4 MFMA row blocks of 16)
constexpr int kRouteWaves = 4;         // tokens per route workgroup (one wave each)
constexpr int kBinThreads = 1024;      // binning runs in one workgroup (16 waves)
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kWitnessValue = 0x950950;
constexpr int kMaxXcds = 64;           // XCDs a launch's task order may be split over
constexpr int kRouterMaxWaves = 8;        // waves of a router-GEMM workgroup (they split its input chunk)
constexpr int kRouterTargetGroups = 256;  // router-GEMM workgroups wanted: one per CU
constexpr int kRouterMaxSplit = 4;        // input chunks (partial sums) per logit at most
// Automatic activation layout of the grouped arm (pairs per woken expert, closed form): h in
// fragment order from kFragMinPairs on, x packed in fragment order from kPackMinPairs on.
constexpr double kFragMinPairs = 8.0;
constexpr double kPackMinPairs = 16.0;

// Routing and binning of a small GEMV-arm batch inside the fused gate/up launch (logits NULL: the
// batch was routed and binned by the routing kernels).  Every workgroup of that launch routes the
// batch before its table fill, bins the pairs, and stores the binned order and the gate/up units
// it reads back (every workgroup stores the same values); workgroup 0 also stores the expert ids,
// the router weights, the down pass's units and, when asked, each pair's binned position, which
// the down pass and the combine read.  (The per-expert counts, offsets and tile map, which no
// later launch of this arm reads, are not stored.)  At most kSmallRouteMaxPairs pairs and
// kFusedRouteMaxTokens tokens; no padded position space.
constexpr int kSmallRouteMaxPairs = 64;
struct SmallRoute {
  const float* logits;  // [n_part][n][E] partial sums added in ascending order, or NULL
  int32_t n_part, n, top_k;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* sorted_pair;
  int32_t* pair_pos;      // NULL, or [n][k]: the binned position of each pair (-1: left out), for TokenCombine
  int32_t unit_pairs[2];  // pairs per decode of the gate/up (0) and down (1) passes
  int32_t* units[2];      // their unit maps (expert, first binned position, pairs)
  int32_t* n_units[2];
};

// The combine folded into the GEMV arm's down pass for a small batch (out NULL: the combine
// kernel runs).  A workgroup task is one token's 16 NT output rows: wave j S + s takes the
// token's pair j (its h row at the pair's binned position) over input blocks [s K/S, (s+1) K/S)
// (S = ksplit), leaving its partial sums in LDS; after a barrier the first wave adds them in
// ascending s, scales each pair's rows, and adds the pairs weighted by their router weights in
// ascending j (the combine's order) into out.
struct TokenCombine {
  const int32_t* topk_idx;  // [n][k] expert of each pair (out of range: the pair is left out)
  const float* topk_w;      // [n][k] router weights
  const int32_t* pair_pos;  // [n][k] binned position of each pair (SmallRoute::pair_pos)
  void* out;                // [n][rows] bf16 or fp32
  int32_t n, k, out_bf16;
};

// One pass of one (or two fused) trellis matrices over binned activation rows.
struct ExpertParams {
  const uint8_t* codes0;        // [E][rows][cols/4]  gate (fused pass) or the single matrix
  const uint8_t* codes1;        // [E][rows][cols/4]  up (fused pass only)
  const uint16_t* scale0;       // [E][rows] fp16
  const uint16_t* scale1;       // [E][rows] fp16 (fused pass only)
  const uint16_t* lut;          // bitshift rung: [65536] fp16 LUT; LUT rung: [512][2] fp16 codebook
  const uint16_t* act;          // [n_act_rows][cols] bf16
  const int32_t* act_row_map;   // activation row of binned position s = map[s] / act_row_div (NULL: s)
  int32_t act_row_div;
  const int32_t* units;         // [n_units][3] (expert, start, len)
  const int32_t* n_units_dev;   // device count of units (NULL: use n_units_host)
  int32_t n_units_host;
  int32_t num_experts;
  int32_t rows, cols;
  int32_t n_pos;                // binned positions are [0, n_pos)
  int32_t n_act_rows;
  void* out;                    // fused: bf16 h [n_pos][rows]; single: fp32 y [n_out_rows][rows]
  const int32_t* out_row_map;   // single pass: output row of position s = map[s] (NULL: s)
  int32_t n_out_rows;
  int32_t n_xcd;                // workgroups are dispatched round-robin over this many XCDs (>= 1)
  const int32_t* unit_pad;      // grouped arm: each unit's start in the padded position space (every expert's
                                // bin rounded up to 16 pairs), or NULL.  When set, the fused pass writes h in
                                // fragment order over padded positions (dense_fragment_offset, rows = padded
                                // positions), the order the down pass reads it in.
  int32_t act_frag;             // with unit_pad: the activations (act) are in that fragment order as well
  int32_t n_pad_max;            // padded positions the fragment-order buffers hold (with unit_pad)
  const uint16_t* dense0;       // dequantize arm: one rows x cols bf16 matrix in fragment order per woken expert, at
                                // its slot (dense_slot) (gate, or the single matrix)
  const uint16_t* dense1;       // dequantize arm: the same for the up weights (fused pass only)
  const int32_t* dense_counts;  // dequantize arm: the per-expert pair counts that define the slots
  int32_t ksplit;               // GEMV arm launched with fewer waves than its configuration's: waves
                                // sharing one task's inputs (a power of 2 dividing cols/128), or <= 1
  SmallRoute route;             // GEMV arm, fused pass: the batch's routing, when logits is set
  TokenCombine tok;             // GEMV arm, down pass: token tasks with the combine, when out is set
};

enum ExpertMode { kModeGateUp = 0, kModeSingle = 1 };
enum ExpertArm { kArmGemv = 0, kArmGrouped = 1, kArmDense = 2 };

struct VariantInfo {
  int waves;             // wave64 per workgroup
  int rows_per_task;     // output rows per wave task (rows must be a multiple of it)
  int pairs_per_decode;  // binned pairs sharing one decode of an expert's rows
  bool input_split;      // GEMV arm: can split a task's inputs over waves (ExpertParams::ksplit)
};
// `variant` in 1..11 (the plan resolves 0).  variant_info returns false for other values.
bool variant_info(int variant, int arm, VariantInfo& v);
// `waves` per workgroup: at most the variant's (VariantInfo::waves); fewer spread a small launch
// over more CUs.
hipError_t launch_expert(int mode, int arm, int variant, int rung, const ExpertParams& p, int grid, int waves,
                         hipStream_t stream);
// The LUT rung's instantiations (their own translation unit, so the two rungs compile in parallel).
hipError_t launch_expert_lut(int mode, int arm, int variant, const ExpertParams& p, int grid, int waves,
                             hipStream_t stream);

// Top-k over logits given as n_part partial sums part[s][t][e] (s-major, n*E apart), added in
// ascending s; n_part = 1 reads plain logits.
// Dequantize-materialise: dense bf16(LUT[state]) (scales not applied) of every row of one or
// two trellis matrices [E][rows][cols/4] into [E][rows][cols] bf16.  expert >= 0 does that
// expert only; otherwise every expert e with counts[e] > 0 (every expert if counts is NULL).
struct DequantParams {
  const uint8_t* codes0;
  const uint8_t* codes1;        // NULL: one matrix
  const uint16_t* lut;
  const int32_t* counts;
  int32_t num_experts, rows, cols, expert;
  uint16_t* out0;
  uint16_t* out1;
  int64_t out_expert_stride;    // elements between slots' matrices in out0/out1 (0: expert-less output); with counts
                                // the woken experts are stored compactly, expert e at slot dense_slot(counts, e)
  int32_t fragment_order;       // 0: row-major [rows][cols]; 1: MFMA fragment order (dense_fragment_offset)
};

// Fragment order of a dense [rows][cols] bf16 matrix, as the dequantize arm's MFMA pass reads
// it: for 16-row block rb, 128-input block kb and MFMA step st, the 64 lanes' 16-byte B
// fragments are contiguous (lane j + 16g holds row 16rb + j, inputs kb*128 + 32g + 8st .. +7).
__host__ __device__ inline size_t dense_fragment_offset(int rb, int kb, int st, int lane, int kblocks) {
  return ((((size_t)rb * kblocks + kb) * 4 + st) * 64 + lane) * 8;
}
hipError_t launch_dequant(const DequantParams& q, int rung, int grid, hipStream_t stream);
hipError_t launch_dequant_lut(const DequantParams& q, int grid, hipStream_t stream);
constexpr int kDequantWaves = 16;

hipError_t launch_route_topk(const float* logits, int32_t n_part, int32_t n, int32_t E, int32_t k,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream);

// Router GEMM (hidden states -> logits).  router_split(n, E, H) is the number S of K chunks
// (a divisor of H/128, at most kRouterMaxSplit) whose partial sums launch_router_gemm writes
// to part[S][n][E]; launch_router_reduce adds them (ascending s) into logits[n][E].
int32_t router_split(int32_t n, int32_t E, int32_t H);
int32_t router_tiles(int32_t n, int32_t E);
int32_t router_waves(int32_t H, int32_t S);
hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w, int32_t n, int32_t E, int32_t H, int32_t S,
                              int32_t n_xcd, float* part, hipStream_t stream);
hipError_t launch_router_reduce(const float* part, int32_t S, int64_t count, float* logits, hipStream_t stream);

// The decode units of the two expert passes (index 0: the fused gate/up pass, 1: the down
// pass): runs of up to unit_pairs[i] pairs of one expert, unit_pairs[i] being that pass
// kernel's pairs per decode (at most kUnitMaxPairs), so every unit is exactly one decode of its
// expert's rows.  map[i]: (expert, first binned position, pairs) per unit, expert-ascending;
// count[i]: the number of units; pad[i]: each unit's first padded position (a multiple of 16),
// or NULL without the padded space.
struct UnitMaps {
  int32_t unit_pairs[2];
  int32_t* map[2];
  int32_t* pad[2];
  int32_t* count[2];
};

// Binning.  units may be NULL (no units); padded_pair/n_pad may be NULL (no padded position
// space).  The padded space rounds every expert's bin up to a multiple of 16 pairs:
// padded_pair[pp] is the pair at padded position pp or -1 in the padding, *n_pad the padded
// total.
hipError_t launch_bin(const int32_t* topk_idx, int32_t n_pairs, int32_t E, int32_t tile_m, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_pair, int32_t* tile_map, int32_t* n_tiles,
                      int32_t* padded_pair, int32_t* n_pad, const UnitMaps* units, hipStream_t stream);

// Batches of at most this many tokens (one per wave of the binning workgroup) are routed and
// binned by one workgroup (launch_route_bin); measured, a second token per wave already costs
// more than the separate launches save.
constexpr int kFusedRouteMaxTokens = kExpertWaves;

// Routing (launch_route_topk) and binning (launch_bin) of n <= kFusedRouteMaxTokens tokens by
// one workgroup, with the same outputs.
hipError_t launch_route_bin(const float* logits, int32_t n_part, int32_t n, int32_t E, int32_t k, int32_t* topk_idx,
                            float* topk_w, int32_t tile_m, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                            int32_t* tile_map, int32_t* n_tiles, int32_t* padded_pair, int32_t* n_pad,
                            const UnitMaps* units, hipStream_t stream);

// Gathers the activation row of every padded position (token = pair / k; padding untouched)
// into fragment order: xs holds n_pad_max padded rows of H bf16 values.
hipError_t launch_pack_act(const uint16_t* x, const int32_t* padded_pair, const int32_t* n_pad, int32_t k,
                           int32_t H, int32_t n_pad_max, uint16_t* xs, hipStream_t stream);

hipError_t launch_combine(const float* y, const float* topk_w, int32_t n, int32_t k, int32_t H, void* out,
                          int out_bf16, hipStream_t stream);

hipError_t launch_witness(int32_t* out, hipStream_t stream);

hipError_t launch_gather_probe(int grid, int32_t rounds, uint32_t* sink, hipStream_t stream);

}  // namespace qtip
