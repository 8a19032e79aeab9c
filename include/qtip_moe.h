/*
 * qtip_moe.h -- C ABI of the MI355X (gfx950) trellis-quantized MoE expert matmul.
 *
 * One MoE layer whose experts are gate/up/down matrices stored as 2-bit
 * bitshift-trellis codes.  Pairs (token, expert) are routed and binned by
 * expert into m-tiles; every woken expert's packed bytes are decoded inside the
 * multiply, so dense weights never exist in memory.
 *
 * Sources (the pages this library implements):
 *  - m-tile occupancy page, PR #167 "gate the trellis grouped GEMM on m-tile
 *    occupancy, not token count": pair binning and the m-tile walk, the fill
 *    formula, the dispatch predicate, the decode-regime floor and the arm pin
 *    (sections "The cause is a threshold", "The fix", "Post-merge note").
 *  - arch-specialise page, PR #99 "arch-specialise the trellis grouped GEMM
 *    (D16) + close the silent-failure holes (D18)": packed 2-bit bytes decoded
 *    in-kernel, contiguous-run decode, status on every launch, empty grid is an
 *    error, unsupported arch is an error, one source of truth for the m-tile
 *    height, an arch witness that never caches a non-answer and declines under
 *    graph capture (sections "The two levers", "D18", "The arch witness").
 *  - prefill page, PR #196: per-arm launch counters and the variant knob where
 *    an unknown value warns and keeps the default ("Two things that were built,
 *    correct, and switched off").
 *
 * Conventions.
 *  - Every pointer is a DEVICE pointer unless the comment says "host".
 *    All device buffers are owned by the caller; the library never allocates,
 *    frees or synchronises inside qtip_moe_forward / qtip_moe_route /
 *    qtip_expert_matmul.  Work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream) and completes asynchronously.
 *  - Every call returns a qtip_status.  A call that returns QTIP_OK has
 *    enqueued work that writes every element of its outputs; no call returns
 *    QTIP_OK after a failed launch (launch status is read back with
 *    hipGetLastError after each launch, mapped to QTIP_ERR_HIP, and the HIP
 *    error text is available from qtip_last_error_detail()).
 *  - bf16 and fp16 values are passed as their 16-bit patterns.
 *
 * Weight formats (readings of the pages, which give only "packed 2-bit bytes" and name two
 * rungs, the bitshift rung "qtip2b" and the LUT rung "qtip2"):
 *  - A matrix with `rows` outputs and `cols` inputs is `rows` independent rows
 *    of cols/4 bytes.  Symbol c of a row = bits [2(c%4), 2(c%4)+2) of byte c/4; the row's
 *    stream bits are its bytes' bits, little-endian, read circularly.
 *  - Storage: a matrix's rows x cols/4 bytes are stored block-interleaved, the 32 bytes of rows
 *    16b..16b+15 for inputs [128k, 128k+128) together: byte 32k + c of row r (c < 32) is at
 *    byte ((r/16) (cols/128) + k) 512 + (r%16) 32 + c of the matrix ([rows/16][cols/128][16][32];
 *    a wave's loads of one block then cover four whole 128-byte lines).
 *  - Bitshift rung: the 16-bit state of weight (r, c) is the 8-symbol window starting at c:
 *    state = sum_j sym((c+j) mod cols) * 4^j; weight(r, c) = bf16(lut[state]) * scale[r], with
 *    lut the 65536-entry fp16 table.
 *  - LUT rung: weights come in pairs (2i, 2i+1); the pair's state is the 9 stream bits from bit
 *    4i on (the low 9 bits of the bitshift state of weight 2i), and the pair's two weights are
 *    bf16(cb[state][0]), bf16(cb[state][1]) times scale[r], with cb the 512 x 2 fp16 codebook.
 *  - Either way the fp16 table value is rounded to bf16 (nearest-even), the dot product
 *    accumulates in fp32, and the fp16 per-output-row scale multiplies the fp32 sum.
 *  - Layer: h = silu(x Wg^T) * (x Wu^T) rounded to bf16; y = h Wd^T;
 *    out[t] = sum_{j<k} w[t,j] * y(t, j) in fp32 (j ascending), then cast.
 *  - Routing: the k largest logits of a token in descending order (ties go to
 *    the lower expert index); weights = softmax over those k logits (fp32).
 *    Logits must be finite (not checked).
 */
#ifndef QTIP_MOE_H
#define QTIP_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qtip_status {
  QTIP_OK = 0,
  QTIP_ERR_INVALID_ARG = 1,    /* a null pointer, a bad shape, a too-small workspace */
  QTIP_ERR_INVALID_CONFIG = 2, /* an empty or oversized launch (n <= 0, n > max_tokens, ...) */
  QTIP_ERR_NOT_SUPPORTED = 3,  /* device is not gfx950, or its code object is not in the library */
  QTIP_ERR_HIP = 4,            /* a HIP runtime or launch error; see qtip_last_error_detail() */
  QTIP_ERR_CAPTURING = 5       /* the arch witness cannot be taken on a capturing stream */
} qtip_status;

/* Arms: the fused GEMV (per-pair decode + VALU dot products), the grouped arm (one decode
 * shared by up to 64 binned pairs, MFMA), and the dequantize arm (the woken experts' weights
 * materialised as dense bf16 in the workspace, then an MFMA pass over them). */
enum { QTIP_ARM_AUTO = 0, QTIP_ARM_GEMV = 1, QTIP_ARM_GROUPED = 2, QTIP_ARM_DEQUANT = 3 };
enum { QTIP_OUT_BF16 = 0, QTIP_OUT_F32 = 1 };
enum { QTIP_ACT_AUTO = 0, QTIP_ACT_ROWS = 1, QTIP_ACT_FRAGMENTS = 2 };
/* The two 2-bit rungs (weight formats) of the expert matrices; see "Weight formats" above. */
enum { QTIP_RUNG_BITSHIFT = 0, QTIP_RUNG_LUT = 1 };
/* How a small GEMV-arm batch is launched (qtip_moe_desc.small_batch). */
enum { QTIP_SMALL_BATCH_FUSED = 0, QTIP_SMALL_BATCH_SEPARATE = 1 };
#define QTIP_LUT_RUNG_BITS 9 /* pair-state bits of the LUT rung: a 2^9 x 2 codebook */

/* Decode-regime floor of the pages: n <= 8 tokens always take the GEMV arm (m-tile page, "The
 * fix": kept there as a graph-capture safety rule, not a performance claim).  The plan-free
 * qtip_fill_* functions below use it. */
#define QTIP_DECODE_REGIME_MAX_TOKENS 8
/* The floor a plan uses by default (qtip_moe_desc.decode_floor = 0), per rung: re-derived for
 * these kernels on MI355X, where both arms are safe under graph capture.  The measured crossover
 * of the V4 layer lies between 7 and 8 tokens on the bitshift rung and between 4 and 5 on the LUT
 * rung (the grouped arm is faster from 8 and from 5). */
#define QTIP_DEFAULT_DECODE_FLOOR_BITSHIFT 7
#define QTIP_DEFAULT_DECODE_FLOOR_LUT 4
/* Default m-tile height: the M of one bf16 MFMA (v_mfma_f32_16x16x32_bf16). */
#define QTIP_DEFAULT_TILE_M 16
/* The fill threshold re-derived for these kernels on MI355X.  The grouped arm decodes each
 * expert once per up to 48-64 binned pairs (not once per m-tile), so tile fill amortises
 * nothing; the measured GEMV/grouped crossover lies between 4 and 7 tokens at V4 routing, where
 * pairs per woken expert are about 1.  At this threshold (1 pair) the fill predicate holds for
 * every n, so the plan's decode floor alone places the switch; the predicate decides with a
 * higher threshold (16 reproduces the pages' gate at 683 tokens). */
#define QTIP_DEFAULT_DISPATCH_TILE_M 1
/* Fused GEMV vs dequantize arm: the GEMV streams an expert's packed bytes once per pair;
 * materialising writes and re-reads dense bf16, 2 x 16/2 = 16 times the packed bytes (m-tile
 * page, "Tests": the constant, and the rule that it must not leave a dequantize window below
 * the grouped boundary). */
#define QTIP_DEFAULT_DEQUANT_TRAFFIC_RATIO 16
/* One decode of an expert's weights is shared by up to this many binned pairs. */
#define QTIP_UNIT_MAX_PAIRS 64
/* Inputs per K block: H and I must be multiples of this; rows a multiple of 16. */
#define QTIP_K_BLOCK 128

typedef struct qtip_moe_desc {
  int32_t num_experts;  /* E >= 1 (<= 1024) */
  int32_t top_k;        /* k, 1 <= k <= E (<= 32) */
  int32_t hidden;       /* H: gate/up inputs and down outputs; multiple of 128 */
  int32_t inter;        /* I: gate/up outputs and down inputs; multiple of 128 */
  int32_t max_tokens;   /* largest n a forward accepts (sizes the workspace), >= 1 */
  int32_t arm_override; /* QTIP_ARM_AUTO (predicate), _GEMV, _GROUPED or _DEQUANT (pins the arm) */
  int32_t variant;      /* expert kernel configuration 1..11 for both passes (10 is a down-pass
                           shape: with it the grouped arm's fused pass runs 9), or 0 = chosen per
                           arm, pass and n by the plan (qtip_moe_plan_schedule reports it);
                           unknown: warning, 0 kept */
  int32_t out_dtype;    /* QTIP_OUT_BF16 or QTIP_OUT_F32 */
  int32_t tile_m;       /* m-tile height of the tile map: 0 = default (16, the MFMA M); else 16, 32, 64 */
  int32_t dispatch_tile_m; /* the fill predicate's threshold in pairs per woken expert: 0 = the value
                              re-derived for these gfx950 kernels (QTIP_DEFAULT_DISPATCH_TILE_M);
                              16 reproduces the pages' sm80 gate; 1..1024 accepted */
  int32_t dequant_traffic_ratio; /* AUTO dispatch keeps the fused GEMV while pairs per woken expert
                              are below this, and sends fills in [ratio, dispatch_tile_m) past the
                              decode floor to the dequantize arm: 0 = 16; 1..1024 accepted.  A plan
                              that can take the dequantize arm (that window is not empty, or the
                              override pins it) holds the dense bf16 weights of every expert a
                              forward can wake in its workspace: 3 x min(E, max_tokens x k) x H x I x
                              2 bytes, and needs H x I < 2^31. */
  int32_t act_layout;   /* grouped arm's activation layout: QTIP_ACT_AUTO (by the closed-form pairs per
                           woken expert), QTIP_ACT_ROWS (gathered rows) or QTIP_ACT_FRAGMENTS (every
                           expert's bin padded to 16 pairs and stored in MFMA fragment order: h always,
                           x packed by an extra pass) */
  int32_t rung;         /* weight format of the experts: QTIP_RUNG_BITSHIFT (a 16-bit window per weight into
                           the 65536-entry LUT) or QTIP_RUNG_LUT (a 9-bit state per weight pair into the
                           512 x 2 codebook); see the weight formats above */
  int32_t decode_floor; /* AUTO dispatch sends n <= decode_floor to the GEMV arm whatever the fill: 0 = the
                           value measured for these kernels and the rung (QTIP_DEFAULT_DECODE_FLOOR_*); 8
                           reproduces the pages' floor; 1..1024 accepted */
  int32_t small_batch;  /* QTIP_SMALL_BATCH_FUSED: a GEMV-arm batch of at most 16 tokens and 64 pairs is routed
                           and binned inside the fused gate+up launch (every workgroup routes it before its
                           table fill; one of them stores the routing for the later launches), which saves
                           the routing launch; and where its down pass fits one round of workgroup tasks on
                           the GPU (one task per token and 16-row block: a single token at H = 4096) and k x
                           the pass's input split fits a workgroup, the combine runs inside the down launch
                           (the token's k pairs summed in ascending j), which saves the combine launch too.
                           QTIP_SMALL_BATCH_SEPARATE: the routing and the combine kernels.  Same arithmetic
                           in the same order either way; the down pass may split its inputs over a different
                           number of waves, which changes the order of its fp32 additions. */
} qtip_moe_desc;

typedef struct qtip_moe_plan_s* qtip_moe_plan_t;

typedef struct qtip_moe_weights {
  const uint8_t* codes_gate;  /* [E][I][H/4] packed 2-bit codes, block-interleaved: [E][I/16][H/128][16][32] */
  const uint8_t* codes_up;    /* [E][I][H/4], block-interleaved */
  const uint8_t* codes_down;  /* [E][H][I/4], block-interleaved: [E][H/16][I/128][16][32] */
  const uint16_t* scale_gate; /* [E][I] fp16, one per output row */
  const uint16_t* scale_up;   /* [E][I] fp16 */
  const uint16_t* scale_down; /* [E][H] fp16 */
  const uint16_t* lut;        /* bitshift rung: [65536] fp16 LUT; LUT rung: [512][2] fp16 codebook; finite */
} qtip_moe_weights;

/* Launch counters of a plan (prefill page, PR #196, "Two things that were built, correct, and
 * switched off": a harness that reports a per-variant timing must show the counter of the
 * variant it claims advancing and the others not; the counters are read by qtip_moe_stats). */
#define QTIP_VARIANT_SLOTS 12 /* index = kernel configuration 1..11 (0 unused) */
typedef struct qtip_moe_stats_s {
  uint64_t forward_calls;     /* successful qtip_moe_forward calls */
  uint64_t gemv_launches;     /* expert-matrix kernel launches on the GEMV arm */
  uint64_t grouped_launches;  /* expert-matrix kernel launches on the grouped arm */
  uint64_t route_launches;    /* routing / binning kernel launches */
  uint64_t combine_launches;  /* combine kernel launches */
  uint64_t router_launches;   /* router GEMM launches (qtip_moe_forward_hidden, qtip_moe_router_logits) */
  uint64_t dequant_launches;  /* dequantize arm: materialise launches and dense expert-pass launches */
  int32_t last_arm;           /* arm taken by the last forward (QTIP_ARM_GEMV / _GROUPED / _DEQUANT) */
  int32_t last_n_tokens;      /* n of the last forward */
  uint64_t gemv_variant_launches[QTIP_VARIANT_SLOTS];    /* GEMV-arm expert launches per configuration */
  uint64_t grouped_variant_launches[QTIP_VARIANT_SLOTS]; /* grouped-arm expert launches per configuration */
  uint64_t routed_in_gate_up; /* forwards whose batch was routed and binned inside the gate+up launch */
  uint64_t combined_in_down;  /* forwards whose combine ran inside the down launch */
} qtip_moe_stats_t;

/* ---- plan -------------------------------------------------------------------------
 * qtip_moe_plan: validate `desc` (host) for `device`, fix the m-tile height and the
 * workspace size, and return a plan (host memory only; launches nothing, so it is safe
 * inside graph capture).  Checks: 1 <= k <= E <= 1024, k <= 32, H and I multiples of
 * 128, max_tokens >= 1, a known arm/out_dtype, tile_m in {0,16,32,64}, max_tokens x k x
 * max(H, I) and the 16-padded pairs x max(H, I) below 2^30 (activation buffers), and the
 * device arch reported by HIP is gfx950 (else QTIP_ERR_NOT_SUPPORTED).  Free with
 * qtip_moe_plan_destroy.  Not thread-safe per plan object (counters).
 * Source: arch-specialise page, PR #99, "D18": an unsupported device is refused instead of
 * running compiled-out code, and the m-tile height has one source of truth that the router,
 * the kernels and the predicate all read (here: the plan); m-tile page, PR #167, "The fix":
 * the dispatch inputs are host scalars, so planning is capture-safe. */
qtip_status qtip_moe_plan(const qtip_moe_desc* desc /*host*/, int device, qtip_moe_plan_t* out /*host*/);

/* Same as qtip_moe_plan for an explicit arch name (e.g. "gfx950:sramecc+:xnack-"),
 * without querying a device: lets host-only callers validate a configuration.  Any other
 * arch is QTIP_ERR_NOT_SUPPORTED (arch-specialise page, PR #99, "D18"). */
qtip_status qtip_moe_plan_for_arch(const qtip_moe_desc* desc /*host*/, const char* gcn_arch_name /*host*/,
                                   qtip_moe_plan_t* out /*host*/);

/* Frees a plan (host memory and any profiling events).  NULL is accepted. */
qtip_status qtip_moe_plan_destroy(qtip_moe_plan_t plan);

/* What the kernels will use: the m-tile height, the workspace bytes a forward needs at
 * max_tokens, and the smallest n for which the predicate (with the plan's dispatch_tile_m)
 * selects the grouped arm.  Any output pointer may be NULL.
 * Source: m-tile page, PR #167, "Tests" (the reported boundary is the exact flip point of the
 * predicate) and arch-specialise page, "D18" (callers read the m-tile height the kernels use
 * from the same place the kernels do). */
qtip_status qtip_moe_plan_info(qtip_moe_plan_t plan, int32_t* tile_m /*host*/, size_t* workspace_bytes /*host*/,
                               int32_t* min_tokens_grouped /*host*/);

/* The expert-kernel schedule a forward of n tokens launches (the arm and, for each of the two
 * expert passes, the kernel configuration and its shape), so callers and benchmarks read what
 * runs.  Source: prefill page, PR #196, "Two things that were built, correct, and switched off"
 * (the selected variant is printed next to every result; a variant that cannot be reached is a
 * defect) and arch-specialise page, "D18" (one source of truth for the tile height). */
typedef struct qtip_moe_kernel_shape {
  int32_t variant;             /* kernel configuration 1..11 actually launched */
  int32_t waves_per_workgroup; /* wave64 per (persistent, one-per-CU) workgroup */
  int32_t rows_per_task;       /* output rows each wave decodes per task (16, 32 or 64) */
  int32_t pairs_per_decode;    /* binned pairs of one expert that share one decode of its rows */
} qtip_moe_kernel_shape;
typedef struct qtip_moe_schedule {
  int32_t arm;                  /* QTIP_ARM_GEMV, QTIP_ARM_GROUPED or QTIP_ARM_DEQUANT */
  int32_t tile_m;               /* m-tile height of the tile map and the predicate */
  qtip_moe_kernel_shape gate_up; /* the fused gate+up pass */
  qtip_moe_kernel_shape down;    /* the down pass */
  int32_t route_in_gate_up;      /* 1: the batch is routed and binned inside the gate+up launch
                                    (qtip_moe_desc.small_batch), 0: by the routing kernels */
  int32_t combine_in_down;       /* 1: the combine runs inside the down launch, 0: its own kernel */
} qtip_moe_schedule;
qtip_status qtip_moe_plan_schedule(qtip_moe_plan_t plan, int32_t n_tokens, qtip_moe_schedule* out /*host*/);

/* The arm a forward of n tokens takes: the override if one is set, else the three-arm closed
 * form (qtip_fill_select_arm) with the plan's dispatch_tile_m, dequant_traffic_ratio and decode_floor.
 * Returns QTIP_ARM_GEMV, QTIP_ARM_GROUPED or QTIP_ARM_DEQUANT, or -1 for a bad plan/n.
 * Source: m-tile page, PR #167, "The fix" (the predicate and the floor) and its post-merge
 * note (an explicit arm pin overrides the predicate, so a harness can A/B the kernels). */
int32_t qtip_moe_select_arm(qtip_moe_plan_t plan, int32_t n_tokens);

/* The pure closed-form predicate for the plan's routing shape: 1 if n > the plan's decode_floor
 * and the expected
 * pairs per woken expert, n k / (E (1 - (1 - k/E)^n)), reach the plan's dispatch_tile_m,
 * else 0; -1 for a bad plan or n < 1.  The plan's arm override is NOT applied here (the arm a
 * forward takes is qtip_moe_select_arm).  Host only; the same header-only code as the plan.
 * Source: m-tile page, PR #167, "The fix" (grouped_gemm_tiles_amortize: an average m-tile is
 * full; the decode-regime floor stays) and "Tests" (the predicate unit-tested at n and n-1). */
int32_t qtip_moe_select_grouped(qtip_moe_plan_t plan, int32_t n_tokens);

/* The token counts [*n_lo, *n_hi) within [1, max_tokens] that the automatic dispatch sends to
 * the dequantize arm (empty, 0 and 0, when dispatch_tile_m <= dequant_traffic_ratio: the m-tile
 * page's "Tests" section requires the two boundaries to leave no such window). Host only;
 * NULL -> INVALID_ARG. */
qtip_status qtip_moe_dequant_range(qtip_moe_plan_t plan, int32_t* n_lo /*host*/, int32_t* n_hi /*host*/);

/* The dequantize arm's first step alone (also a dense reference of the decode): writes
 * bf16(LUT[state]) of every weight of one expert's matrix (0 = gate [I][H], 1 = up [I][H],
 * 2 = down [H][I]; scales not applied) to dense_out (device, row-major, 16-byte aligned).
 * Errors: NULL, matrix or expert out of range, misalignment -> INVALID_ARG; launch -> HIP.
 * Source: m-tile page, PR #167, "Tests" (the dequantize-materialize path, the third arm). */
qtip_status qtip_moe_dequantize(qtip_moe_plan_t plan, const qtip_moe_weights* w /*host struct of device ptrs*/,
                                int32_t matrix, int32_t expert, void* dense_out, void* stream);

/* ---- closed-form fill model (m-tile page, "The cause is a threshold" and "The fix") --
 * Uniform routing of n tokens to k of E experts wakes E(1-(1-k/E)^n) experts on average;
 * pairs per woken expert = n k / that.  The grouped arm is selected iff n > 8 (the pages'
 * floor, QTIP_DECODE_REGIME_MAX_TOKENS; a plan uses its own decode_floor) and pairs per woken
 * expert >= tile_m (the threshold).  Pure host functions of their arguments. */
double qtip_fill_woken_experts(int32_t n, int32_t k, int32_t E);
double qtip_fill_pairs_per_woken_expert(int32_t n, int32_t k, int32_t E);
int32_t qtip_fill_select_grouped(int32_t n, int32_t k, int32_t E, int32_t tile_m); /* 1 / 0, -1 bad args */
int32_t qtip_fill_min_tokens(int32_t k, int32_t E, int32_t tile_m);                /* smallest n selected */
/* Three-arm dispatch: QTIP_ARM_GROUPED if qtip_fill_select_grouped; else QTIP_ARM_GEMV if n <= 8
 * or pairs per woken expert < dequant_ratio; else QTIP_ARM_DEQUANT.  -1 for bad arguments. */
int32_t qtip_fill_select_arm(int32_t n, int32_t k, int32_t E, int32_t tile_m, int32_t dequant_ratio);

/* ---- forward ----------------------------------------------------------------------
 * One MoE layer for n tokens: route, bin, gate+up (SwiGLU), down, combine.
 * Source: m-tile page, PR #167, "The cause is a threshold" (pairs sorted by expert and walked
 * as sum_e ceil(count_e / tile_m) m-tiles; the per-pair GEMV for low fill); arch-specialise
 * page, PR #99, "The two levers" (packed 2-bit bytes decoded inside the multiply, runs of 32
 * symbols seeded from their window; fewer decodes per expert) and "D18" (status of every
 * launch; an empty launch is an error; no success with an unwritten output); step page, PR
 * #202, "Ruled out by reading" (the weighted per-token combine of the expert outputs).
 *   x        [n][H] bf16 activations;   logits [n][E] fp32 router logits
 *   out      [n][H] bf16 or fp32 (plan's out_dtype); every element is written
 *   workspace >= qtip_moe_plan_info(...).workspace_bytes bytes, 256-byte aligned,
 *            contents need no initialisation; must not overlap inputs or out.
 * Errors: NULL plan/weights/x/logits/out/workspace -> INVALID_ARG; n <= 0 or
 * n > max_tokens -> INVALID_CONFIG (an empty launch is an error, not a no-op);
 * workspace too small or misaligned -> INVALID_ARG; device not gfx950 or witness
 * failed -> NOT_SUPPORTED; first call on a device while `stream` is capturing ->
 * CAPTURING; launch failure -> HIP.  Bumps the per-arm launch counters. */
qtip_status qtip_moe_forward(qtip_moe_plan_t plan, const qtip_moe_weights* w /*host struct of device ptrs*/,
                             const void* x_bf16, const float* logits, int32_t n_tokens, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- the forward without allocation -----------------------------------------------------
 * For callers that cannot allocate: code under HIP graph capture that may not call hipMalloc,
 * tight serving loops, and harnesses that forbid allocation.  The same layer as
 * qtip_moe_forward (same kernels, same results bit for bit), with its scratch in a device
 * array that the library holds for the life of the process, QTIP_NOALLOC_SCRATCH_BYTES per
 * GPU it runs on, instead of a caller workspace.  The caller still passes inputs and outputs.
 *   The scratch is laid out for this call's n_tokens, so a call fits when the layer needs at
 *   most QTIP_NOALLOC_SCRATCH_BYTES for n tokens: the V4 layer (E=256, top-6, H=4096,
 *   I=2048) up to 405 tokens (534 with the GEMV arm pinned), the tiny layer at any n.  A call
 *   that takes the dequantize arm (the woken experts' dense weights) does not fit at V4 sizes.
 *   Makes no allocation, no free and no synchronisation on any call; the first call on a
 *   device looks up that device's scratch address (and takes the arch witness, as
 *   qtip_moe_forward does), so make it once outside capture.  The scratch needs no
 *   initialisation: every call writes what it reads.
 *   All calls on one GPU share that GPU's scratch: calls that overlap on one GPU (two
 *   streams, two threads, two plans) race and must be serialised by the caller.
 * Errors: as qtip_moe_forward; a layer that needs more scratch than the maximum for n tokens
 * -> QTIP_ERR_INVALID_CONFIG (checked on the host before any device work). */
#define QTIP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
qtip_status qtip_moe_forward_noalloc(qtip_moe_plan_t plan, const qtip_moe_weights* w /*host struct of device ptrs*/,
                                     const void* x_bf16, const float* logits, int32_t n_tokens, void* out,
                                     void* stream);

/* ---- router GEMM (794-ms-decode-step page, PR #202, closing list of remaining
 * un-owned items, item (3): the router GEMM ahead of top-k, moved from FP32 scalar
 * cores to the matrix units) ---------------------------------------------------------
 * logits[t][e] = sum_h x[t][h] * w_router[e][h]: bf16 operands (both row-major, rows of
 * H), fp32 accumulation on v_mfma_f32_16x16x32_bf16, no bias.  The sum over h is split
 * into S = qtip_moe_router_split(plan, n) chunks of H/S inputs (a divisor of H/128 chosen
 * from n, E and H only); each chunk is summed on the matrix cores and the chunks are added
 * in ascending order, so for a given n both entry points below produce bit-identical
 * logits.  Any order of fp32 additions errs by at most 2 H 2^-24 sum_h |x w| (per logit).
 *
 * qtip_moe_router_logits: writes logits [n][E] fp32 (device).  x [n][H] and w_router [E][H]
 *   are device bf16, 16-byte aligned; the workspace is the forward's (same size rule).
 *   Errors as qtip_moe_forward (NULL -> INVALID_ARG, n out of [1, max_tokens] ->
 *   INVALID_CONFIG, small or misaligned workspace -> INVALID_ARG, launch -> HIP).
 * qtip_moe_forward_hidden: the layer of qtip_moe_forward with its logits computed by the
 *   router GEMM from x (the logits stay in the workspace); out equals
 *   qtip_moe_forward(x, qtip_moe_router_logits(x)) bit for bit.  Errors as
 *   qtip_moe_forward; w_router NULL or misaligned -> INVALID_ARG.
 * qtip_moe_router_split: S for n tokens, or -1 for a bad plan/n (host only). */
qtip_status qtip_moe_router_logits(qtip_moe_plan_t plan, const void* x_bf16, const void* w_router_bf16,
                                   int32_t n_tokens, float* logits, void* workspace, size_t workspace_bytes,
                                   void* stream);
qtip_status qtip_moe_forward_hidden(qtip_moe_plan_t plan, const qtip_moe_weights* w /*host struct of device ptrs*/,
                                    const void* w_router_bf16, const void* x_bf16, int32_t n_tokens, void* out,
                                    void* workspace, size_t workspace_bytes, void* stream);
int32_t qtip_moe_router_split(qtip_moe_plan_t plan, int32_t n_tokens);

/* ---- routing and binning alone (bit-exact testing of the routing launcher) ----------
 * Source: m-tile page, PR #167, "The cause is a threshold": (token, expert) pairs sorted by
 * expert and cut into m-tiles of at most tile_m pairs, sum_e ceil(count_e / tile_m) of them;
 * the workload definition's router (softmax over the top-k logits).
 *   topk_idx [n][k] int32, topk_w [n][k] fp32, counts [E], offsets [E+1] (exclusive
 *   scan, offsets[E] = n k), sorted_pair [n k] (pair ids p = t k + j grouped by expert,
 *   ascending p inside each expert), tile_map [n k][3] int32 (expert, start, len) tiles
 *   in ascending expert order, len <= tile_m; n_tiles [1] = sum_e ceil(count_e/tile_m).
 *   Rows of tile_map past n_tiles are left unwritten.  Errors as qtip_moe_forward. */
qtip_status qtip_moe_route(qtip_moe_plan_t plan, const float* logits, int32_t n_tokens, int32_t* topk_idx,
                           float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                           int32_t* tile_map, int32_t* n_tiles, void* stream);

/* ---- one trellis matrix times binned activation rows ------------------------------
 * The expert matmul by itself (arch-specialise page, PR #99, "The two levers": packed codes
 * decoded in-kernel and multiplied; used for per-matrix timing and the bit-exact decode test).
 * It walks a unit map rather than a tile map: a unit is (expert, first binned row, pairs) with
 * up to 64 pairs, which one decode of the expert's rows serves.  Any m-tile map of
 * qtip_moe_route (tiles of at most tile_m <= 64 pairs) is a valid unit map, so a tile map can
 * be passed as it is; num_experts and n_rows_a bound the map's entries on the device.
 * For each unit u < n_units of unit_map [n_units][3] = (expert e, start s, len L):
 *   y[s+i][r] = scale[e][r] * sum_c a[s+i][c] * bf16(lut[state_e(r, c)])   (i < L, r < rows)
 *   codes [E][rows][cols/4] (block-interleaved, see the weight formats above; the plan's rung),
 *   scales [E][rows] fp16, lut [65536] fp16 (LUT rung: [512][2] codebook),
 *   a [n_rows_a][cols] bf16, y [n_rows_a][rows] fp32.
 * `arm` is QTIP_ARM_GEMV or QTIP_ARM_GROUPED.  Constraints: rows % 16 == 0, cols % 128
 * == 0, n_rows_a x cols < 2^30, 1 <= L <= 64, 0 <= e < num_experts, 0 <= s, s + L <= n_rows_a.  A unit that
 * violates them on the device is skipped (its rows of y are not written), so device-side
 * garbage cannot cause out-of-bounds access.  Rows of y no unit covers are not written.
 * n_units == 0 is INVALID_CONFIG. */
qtip_status qtip_expert_matmul(qtip_moe_plan_t plan, int32_t arm, const uint8_t* codes, const uint16_t* scales,
                               const uint16_t* lut, int32_t num_experts, int32_t rows, int32_t cols,
                               const void* a_bf16, int32_t n_rows_a, const int32_t* unit_map, int32_t n_units,
                               float* y, void* stream);

/* ---- observability -----------------------------------------------------------------
 * qtip_moe_stats: copies the plan's launch counters (per arm, and per kernel configuration
 * on the GEMV and grouped arms) into *out; qtip_moe_stats_reset zeroes them.  Host only.
 * Source: prefill page, PR #196, "Two things that were built, correct, and switched off" (a
 * per-variant timing must come with the launch counter of that variant advancing, and only
 * that one). */
qtip_status qtip_moe_stats(qtip_moe_plan_t plan, qtip_moe_stats_t* out /*host*/);
qtip_status qtip_moe_stats_reset(qtip_moe_plan_t plan);

/* One line naming the arm the plan takes for n tokens (GEMV, grouped or dequantize), the mean
 * m-tile fill, pairs per woken expert and the boundary n, so a results artifact can be read
 * back to the dispatch that produced it.  Writes at most buf_len bytes including the NUL.
 * Source: m-tile page, PR #167, "Tests" (the engagement log) and "Re-measurement on this
 * branch" (the line: tokens x top-k of E, m-tile fill %, pairs per woken expert against the
 * m-tile height, the boundary n of the routing shape). */
qtip_status qtip_moe_engaged_line(qtip_moe_plan_t plan, int32_t n_tokens, char* buf /*host*/, size_t buf_len);

/* Writes the engagement line (qtip_moe_engaged_line) for n tokens to stderr once per plan and
 * arm: the first call for the arm that n selects prints it and sets *printed = 1 (if printed is
 * not NULL); later calls for the same arm print nothing and set *printed = 0.  Host only;
 * errors as qtip_moe_engaged_line.  Source: m-tile page, PR #167, "Tests" (runs log which MoE
 * kernel was selected and at what tile fill, once) and "Re-measurement on this branch". */
qtip_status qtip_moe_log_engaged(qtip_moe_plan_t plan, int32_t n_tokens, int32_t* printed /*host*/);

/* Take (once per device, cached only on success) the arch witness: a one-thread kernel
 * from this library's gfx950 code object writes a known value that is read back.  Fails
 * with CAPTURING if `stream` is capturing, NOT_SUPPORTED if the value is wrong or the
 * kernel cannot run.  qtip_moe_forward / _route / qtip_expert_matmul call it on first use.
 * Source: arch-specialise page, PR #99, "The arch witness" (never cache a non-answer; decline
 * under graph capture rather than launch a probe into the capture). */
qtip_status qtip_arch_witness(int device, void* stream);

/* Per-stage timing (prefill page, PR #196: a measurement is only believed when a second
 * instrument agrees; these events are checked against the profiler's kernel times).
 * qtip_moe_profile_enable(plan, capacity) creates capacity x 6 HIP events
 * (capacity <= 4096; 0 disables and frees them); every later forward on the plan records an
 * event before its first kernel and after each of its five kernels (route, bin, gate+up,
 * down, combine) on the forward's stream, cycling through `capacity` slots.  Batches of up to
 * 16 tokens are routed and binned by one kernel: their "route" stage holds both and their
 * "bin" stage only the activation packing, if any (the "bin" stage always includes it).
 * qtip_moe_profile_read waits for the recorded events, writes the summed milliseconds per
 * stage over the last min(forwards, capacity) forwards into stage_ms[5] (host), their count
 * into n_forwards, and clears the record.  Enabling creates events, so do it outside capture. */
#define QTIP_PROFILE_STAGES 5
qtip_status qtip_moe_profile_enable(qtip_moe_plan_t plan, int32_t capacity);
qtip_status qtip_moe_profile_read(qtip_moe_plan_t plan, double* stage_ms /*host [5]*/, int32_t* n_forwards /*host*/);

/* Decode-ceiling calibration (a diagnostic of this implementation, not part of the forward path
 * and not taken from the pages).  The trellis decode
 * is bound by uniformly random 2-byte gathers from the 65536-entry LUT held in LDS; this runs
 * that gather alone on the current device (one 1024-thread workgroup per CU, 128 KiB LDS table,
 * 16 gathers per lane per round at pseudo-random addresses, `rounds` rounds) and reports the
 * measured lookups per second.  sink: device buffer of at least (CU count x 1024) uint32 that
 * receives per-thread checksums (keeps the gathers live); its contents are meaningless.
 * Synchronises the stream.  rounds in [1, 1 << 20]. */
qtip_status qtip_measure_lut_gather(int32_t rounds, uint32_t* sink, size_t sink_elems, void* stream,
                                    double* lookups_per_second /*host*/);

/* Status names and error text (arch-specialise page, PR #99, "D18": every launch status is read
 * back and surfaced, never swallowed).  qtip_status_string returns a static name
 * ("QTIP_ERR_UNKNOWN" for a value outside the enum); qtip_last_error_detail returns the text of
 * the last error raised on the calling thread ("" if none), valid until that thread's next call. */
const char* qtip_status_string(qtip_status s);
const char* qtip_last_error_detail(void);

#ifdef __cplusplus
}
#endif
#endif /* QTIP_MOE_H */
