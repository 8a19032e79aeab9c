// C ABI of the trellis MoE expert path: plans, dispatch, status mapping, witness, counters.
//
// Interface rules follow the arch-specialise page (PR #99, section "D18 -- this path had
// no launch-status check anywhere" and "The arch witness"): every launch's status is read
// back and mapped to an error, an empty grid is an error rather than a silent no-op, an
// unsupported device is refused instead of running compiled-out code, the m-tile height
// comes from one place (the plan) for the router, the kernels and the predicate, and the
// witness declines under graph capture and caches only a successful answer.  The variant
// knob follows the prefill page (PR #196): an unknown value warns and keeps the default.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qtip_moe.h"
#include "fill_predicate.h"
#include "qtip_internal.h"

using namespace qtip;

struct qtip_moe_plan_s {
  qtip_moe_desc d;
  int32_t tile_m;
  int32_t dispatch_tile_m;
  int32_t decode_floor;         // n <= decode_floor always takes the GEMV arm
  int32_t dequant_ratio;        // fused GEMV kept while pairs per woken expert are below this
  int32_t dequant_lo, dequant_hi;  // token counts [lo, hi) the automatic dispatch sends to the dequantize arm
  bool dense;                   // the dequantize arm may run: its dense weights are in the workspace
  bool frag;                    // the grouped arm may use the fragment-order layout (padded space, h)
  bool pack;                    // ... and pack x into it (its buffer is in the workspace)
  int32_t device;  // -1: created from an arch name; the current device is used at call time

  int32_t min_tokens_grouped;
  size_t ws_bytes;
  qtip_moe_stats_t stats;
  bool engaged_logged[4] = {false, false, false, false};  // qtip_moe_log_engaged: printed per arm
  // per-stage timing ring (qtip_moe_profile_enable)
  std::vector<hipEvent_t> prof_events;  // capacity x (kStages + 1)
  int32_t prof_capacity = 0;
  int64_t prof_recorded = 0;            // forwards recorded since the last read
};

namespace {
constexpr int kStages = QTIP_PROFILE_STAGES;

void prof_free(qtip_moe_plan_s* p) {
  for (hipEvent_t e : p->prof_events) (void)hipEventDestroy(e);
  p->prof_events.clear();
  p->prof_capacity = 0;
  p->prof_recorded = 0;
}

// Records boundary `b` (0 = before the first kernel, 1..5 = after stage b) of this forward.
inline hipError_t prof_mark(qtip_moe_plan_s* p, int b, hipStream_t st) {
  if (p->prof_capacity == 0) return hipSuccess;
  const int64_t slot = p->prof_recorded % p->prof_capacity;
  return hipEventRecord(p->prof_events[slot * (kStages + 1) + b], st);
}
}  // namespace

namespace {

// Kernel configuration when the plan's variant is 0, measured on MI355X with V4-shaped layers
// (bench.py --sweep over variants) and chosen from host scalars only, so the choice is safe
// during graph capture.
//  * Grouped arm, by the closed-form pairs per woken expert (ppe).  Fused pass: 16 waves of
//    16-row tasks below 4 (many short tasks keep every CU busy), then 12 waves of 32-row tasks
//    sharing a decode across three 16-pair blocks (each activation fragment feeds more MFMAs,
//    and an expert with up to 48 pairs is decoded once).  Down pass: 16 waves of 32-row tasks
//    below 3, 12 waves of 64-row tasks with 12-byte code loads from 3, sharing a decode across
//    three 16-pair blocks from 4.
//  * GEMV arm, by the expected task count.  Fused pass: 12-wave workgroups of 16-row tasks
//    (inputs split over several waves where the tasks are few) below 14000 32-row tasks
//    (n <= 64 on the V4 layer: 1-11 % ahead of the 8- and 16-wave shapes), 8 waves of 32-row
//    tasks from there.  Down pass: 16-wave workgroups of 16-row tasks up to 6144 32-row tasks
//    (every measured batch of 1 to 8 tokens), 32-row tasks beyond.
// The LUT rung's decode reads one 4-byte codebook entry per two weights, so its passes are
// bound by the vector-memory path (activation fragments above all) rather than by LDS gathers;
// taller tasks, which feed each fragment to more MFMAs, pay there (bench.py --sweep-rung lut
// over variants, n = 1 to 1024):
//  * Grouped arm.  Fused pass: 16 waves of 16-row tasks below 1.15 pairs per woken expert, 12
//    waves of 32-row tasks below 8, 8 waves of 64-row tasks from 8.  Down pass: 12 waves of
//    64-row tasks (two 16-pair blocks per decode) throughout (level with three blocks per
//    decode at n = 1024, ahead below).
//  * GEMV arm.  Fused pass: 12-wave workgroups of 16-row tasks while a 256-CU launch has fewer
//    than 5 of them per CU (their inputs split over several waves; n=1 24 against 27 us with
//    8 waves), 16-wave workgroups of 16-row tasks from there, and 8 waves of 32-row tasks once
//    those give each of the 2048 wave slots of a 256-CU, 8-wave launch one; down pass: 16-wave
//    workgroups of 16-row tasks below
//    1536 32-row tasks (batches of one and two tokens), of 32-row tasks from there.
int kernel_arm(int32_t arm) {
  return arm == QTIP_ARM_GROUPED ? kArmGrouped : (arm == QTIP_ARM_DEQUANT ? kArmDense : kArmGemv);
}

int resolve_variant(const qtip_moe_plan_s* plan, int arm, int mode, int32_t n_tokens) {
  if (arm == kArmDense) return 3;  // the dequantize arm has one configuration
  if (plan->d.variant != kVariantDefault) {
    // variant 10 is a down-pass shape; its fused grouped task would spill, so that pass runs 9
    if (plan->d.variant == 10 && mode == kModeGateUp && arm == kArmGrouped) return 9;
    return plan->d.variant;
  }
  const int32_t E = plan->d.num_experts, k = plan->d.top_k;
  const int32_t n = n_tokens >= 1 ? n_tokens : 1;
  const bool lut = plan->d.rung == QTIP_RUNG_LUT;
  if (arm == kArmGemv) {
    const double rows = mode == kModeGateUp ? plan->d.inter : plan->d.hidden;
    const double woken = fill_woken_experts(n, k, E);
    const double tall_tasks = woken * rows / 32.0;
    if (mode == kModeSingle) {
      if (lut) return tall_tasks < 1536.0 ? 1 : 3;
      return tall_tasks < 6144.0 ? 1 : 4;
    }
    if (!lut) return tall_tasks < 14000.0 ? 11 : 4;
    if (tall_tasks >= 2048.0) return 4;
    return woken * rows / 16.0 >= 5.0 * 256.0 ? 1 : 11;
  }
  const double ppe = fill_pairs_per_woken_expert(n, k, E);
  if (lut) {
    if (mode == kModeGateUp) return ppe < 1.15 ? 1 : (ppe < 8.0 ? 6 : 5);
    return 7;
  }
  if (mode == kModeGateUp) return ppe < 4.0 ? 1 : 9;
  return ppe < 3.0 ? 3 : (ppe < 4.0 ? 7 : 10);
}

// A variant whose task height does not divide `rows` falls back to the next shorter task of the
// same family (64 -> 32 rows), then to the 16-row configuration with the same register budget.
int fit_variant(int variant, int arm, int32_t rows) {
  VariantInfo v{};
  if (!variant_info(variant, arm, v)) return 1;
  if (rows % v.rows_per_task == 0) return variant;
  if (rows % 32 == 0 && v.rows_per_task == 64) return v.waves == 12 ? 6 : 4;
  return v.waves == 8 ? 2 : 1;
}

thread_local std::string g_detail;

qtip_status fail(qtip_status s, const std::string& what) {
  g_detail = what;
  return s;
}

qtip_status hip_fail(hipError_t e, const char* where) {
  g_detail = std::string(where) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
  return QTIP_ERR_HIP;
}

bool arch_is_supported(const char* name) { return name != nullptr && std::strncmp(name, "gfx950", 6) == 0 &&
                                                  (name[6] == '\0' || name[6] == ':'); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t topk_idx, topk_w, counts, offsets, sorted_pair, pair_pos, tile_map, n_tiles, unit_map, n_units, h, y, router_part,
      dense_gate, dense_up, dense_down, padded_pair, unit_pad, n_pad, xs, total;
  size_t max_units;  // entries of each pass's unit map (and unit_pad)
};

// Padded positions (every woken expert's bin rounded up to 16 pairs) for n tokens, a multiple of 16.
size_t pad_positions(const qtip_moe_desc& d, int32_t n_tokens) {
  const size_t P = (size_t)n_tokens * d.top_k;
  const size_t woken_max = P < (size_t)d.num_experts ? P : (size_t)d.num_experts;
  return (P + 15 * woken_max + 15) & ~(size_t)15;
}

// Largest router-GEMM partial buffer, S(n) * n * E floats, over the batch sizes a plan accepts.
// From 32 * kRouterTargetGroups tokens on there are enough tiles for a split of 1, so n_max
// bounds the rest.
size_t router_part_elems(const qtip_moe_desc& d, int32_t n_max) {
  size_t best = (size_t)n_max * (size_t)d.num_experts;
  const int32_t scan = n_max < 32 * kRouterTargetGroups ? n_max : 32 * kRouterTargetGroups;
  for (int32_t n = 1; n <= scan; ++n) {
    const size_t e = (size_t)router_split(n, d.num_experts, d.hidden) * (size_t)n * (size_t)d.num_experts;
    if (e > best) best = e;
  }
  return best;
}

// `dense`, `frag`, `pack`: whether the plan can take the dequantize arm, the fragment layout
// and the packed x; the buffers of what it cannot take are left out.
WsLayout ws_layout(const qtip_moe_desc& d, int32_t tile_m, int32_t n_tokens, bool dense, bool frag, bool pack) {
  const size_t P = (size_t)n_tokens * d.top_k;
  const size_t woken_max = P < (size_t)d.num_experts ? P : (size_t)d.num_experts;
  const size_t max_tiles = P / tile_m + woken_max + 1;
  const size_t max_units = P + woken_max + 1;  // units of one pair at the least (the GEMV arm's)
  WsLayout L{};
  L.max_units = max_units;
  size_t o = 0;
  L.topk_idx = o;     o = align256(o + P * 4);
  L.topk_w = o;       o = align256(o + P * 4);
  L.counts = o;       o = align256(o + (size_t)d.num_experts * 4);
  L.offsets = o;      o = align256(o + ((size_t)d.num_experts + 1) * 4);
  L.sorted_pair = o;  o = align256(o + P * 4);
  L.pair_pos = o;     o = align256(o + P * 4);  // token tasks: each pair's binned position
  L.tile_map = o;     o = align256(o + max_tiles * 12);
  L.n_tiles = o;      o = align256(o + 4);
  L.unit_map = o;     o = align256(o + 2 * max_units * 12);  // one unit map per expert pass
  L.n_units = o;      o = align256(o + 2 * 4);
  const size_t PP = frag ? pad_positions(d, n_tokens) : 0;
  L.h = o;            o = align256(o + (frag ? PP : P) * (size_t)d.inter * 2);  // rows (P) or fragment order (PP)
  L.y = o;            o = align256(o + P * (size_t)d.hidden * 4);
  L.router_part = o;  o = align256(o + router_part_elems(d, n_tokens) * 4);
  // dequantize arm (only when the plan can take it): the dense bf16 weights of at most
  // min(E, n k) woken experts, one slot each
  const size_t dense_mat = dense ? woken_max * (size_t)d.hidden * (size_t)d.inter * 2 : 0;
  L.dense_gate = o;   o = align256(o + dense_mat);
  L.dense_up = o;     o = align256(o + dense_mat);
  L.dense_down = o;   o = align256(o + dense_mat);
  L.padded_pair = o;  o = align256(o + PP * 4);
  L.unit_pad = o;     o = align256(o + (frag ? 2 * max_units * 4 : 0));
  L.n_pad = o;        o = align256(o + 4);
  L.xs = o;           o = align256(o + (pack ? PP * (size_t)d.hidden * 2 : 0));
  L.total = o;
  return L;
}

// Units of at most unit_pairs pairs that n tokens can make: each woken expert's pairs / unit_pairs,
// plus one partial unit.
size_t max_units_for(const qtip_moe_desc& d, int32_t n_tokens, int32_t unit_pairs) {
  const size_t P = (size_t)n_tokens * d.top_k;
  const size_t woken_max = P < (size_t)d.num_experts ? P : (size_t)d.num_experts;
  return P / (size_t)unit_pairs + woken_max;
}

// --- per-device state: CU count and the witness ---------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_witness_ok[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];
std::mutex g_witness_mutex;

qtip_status current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (*dev < 0 || *dev >= kMaxDevices) return fail(QTIP_ERR_NOT_SUPPORTED, "device index out of range");
  return QTIP_OK;
}

qtip_status witness_on(int dev, hipStream_t stream) {
  if (g_witness_ok[dev].load(std::memory_order_acquire)) return QTIP_OK;
  std::lock_guard<std::mutex> lock(g_witness_mutex);
  if (g_witness_ok[dev].load(std::memory_order_acquire)) return QTIP_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return fail(QTIP_ERR_CAPTURING, "arch witness not taken yet and the stream is capturing; call "
                                    "qtip_arch_witness outside capture first");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (!arch_is_supported(prop.gcnArchName))
    return fail(QTIP_ERR_NOT_SUPPORTED, std::string("device arch ") + prop.gcnArchName + " is not gfx950");
  int32_t* buf = nullptr;
  e = hipMalloc(&buf, sizeof(int32_t));
  if (e != hipSuccess) return hip_fail(e, "witness hipMalloc");
  int32_t host = 0;
  e = launch_witness(buf, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(&host, buf, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  (void)hipFree(buf);
  if (e != hipSuccess) {
    g_detail = std::string("arch witness could not run: ") + hipGetErrorName(e);
    return QTIP_ERR_NOT_SUPPORTED;
  }
  if (host != kWitnessValue) return fail(QTIP_ERR_NOT_SUPPORTED, "arch witness returned a wrong value");
  g_cu_count[dev].store(prop.multiProcessorCount, std::memory_order_release);
  g_witness_ok[dev].store(1, std::memory_order_release);
  return QTIP_OK;
}

qtip_status ensure_device(qtip_moe_plan_t plan, hipStream_t stream, int* dev_out) {
  int dev = 0;
  qtip_status s = current_device(&dev);
  if (s != QTIP_OK) return s;
  if (plan->device >= 0 && plan->device != dev)
    return fail(QTIP_ERR_INVALID_ARG, "current device differs from the plan's device");
  s = witness_on(dev, stream);
  if (s != QTIP_OK) return s;
  *dev_out = dev;
  return QTIP_OK;
}

// MI355X dispatches workgroups round-robin over 8 XCDs of 32 CUs; other CU counts are
// treated as one XCD (only the task order, not correctness, depends on this).
int xcd_count(int dev) {
  const int cus = g_cu_count[dev].load(std::memory_order_acquire);
  const int nx = (cus >= 64 && cus % 32 == 0) ? cus / 32 : 1;
  return nx <= kMaxXcds ? nx : 1;
}

int persistent_grid(int dev, size_t max_tasks, int waves) {
  const size_t cus = (size_t)g_cu_count[dev].load(std::memory_order_acquire);
  size_t need = (max_tasks + waves - 1) / waves;
  if (need < 1) need = 1;
  return (int)(need < cus ? need : cus);
}

// Workgroups and waves per workgroup of a persistent expert launch over at most max_tasks
// tasks: one workgroup per CU with the configuration's waves when the tasks fill them.  With
// fewer tasks, the GEMV arm (spread) still takes a workgroup on as many CUs as there are tasks,
// each with fewer waves (a CU's LUT gathers are its own: measured +35 % per layer at one token,
// +7 % at two); the other arms keep full workgroups on fewer CUs.  Where a workgroup would then
// hold few waves, the GEMV arm can also split each task's kblocks input blocks over ksplit waves
// (a power of 2, at least 2 blocks each) to fill its configuration's waves.
struct LaunchShape {
  int grid, waves, ksplit;
};

LaunchShape persistent_shape(int dev, size_t max_tasks, int max_waves, bool spread, bool input_split = false,
                             int kblocks = 1) {
  const size_t cus = (size_t)g_cu_count[dev].load(std::memory_order_acquire);
  if (!spread || max_tasks >= cus * (size_t)max_waves) return {persistent_grid(dev, max_tasks, max_waves), max_waves, 1};
  size_t tpw = (max_tasks + cus - 1) / cus;  // tasks per workgroup
  if (tpw < 1) tpw = 1;
  size_t grid = (max_tasks + tpw - 1) / tpw;
  if (grid < 1) grid = 1;
  if (grid > cus) grid = cus;
  int split = 1;
  while (input_split && tpw * (size_t)(2 * split) <= (size_t)max_waves && kblocks % (2 * split) == 0 &&
         kblocks / (2 * split) >= 2)
    split *= 2;
  return {(int)grid, (int)tpw * split, split};
}

qtip_status validate_desc(const qtip_moe_desc* d, int32_t* tile_m) {
  if (!d) return fail(QTIP_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_experts < 1 || d->num_experts > kMaxExperts)
    return fail(QTIP_ERR_INVALID_ARG, "num_experts must be in [1, 1024]");
  if (d->top_k < 1 || d->top_k > d->num_experts || d->top_k > kMaxTopK)
    return fail(QTIP_ERR_INVALID_ARG, "top_k must be in [1, min(num_experts, 32)]");
  if (d->hidden < kKBlock || d->hidden % kKBlock) return fail(QTIP_ERR_INVALID_ARG, "hidden must be a positive multiple of 128");
  if (d->inter < kKBlock || d->inter % kKBlock) return fail(QTIP_ERR_INVALID_ARG, "inter must be a positive multiple of 128");
  if (d->max_tokens < 1) return fail(QTIP_ERR_INVALID_ARG, "max_tokens must be >= 1");
  if ((int64_t)d->max_tokens * d->top_k > (1 << 24)) return fail(QTIP_ERR_INVALID_ARG, "max_tokens * top_k exceeds 2^24");
  // activation buffers (x: n x H, h: n k x I) are read through buffer resources with 32-bit byte
  // offsets below 2^31 (the offset 2^31 marks a skipped load)
  if ((int64_t)d->max_tokens * d->top_k * (d->hidden > d->inter ? d->hidden : d->inter) >= ((int64_t)1 << 30))
    return fail(QTIP_ERR_INVALID_ARG, "max_tokens * top_k * max(hidden, inter) must be below 2^30");
  if ((int64_t)d->hidden * d->inter / 4 >= ((int64_t)1 << 31))
    return fail(QTIP_ERR_INVALID_ARG, "one expert matrix must be below 2^31 bytes");
  {
    const int64_t P = (int64_t)d->max_tokens * d->top_k;
    const int64_t PP = P + 15 * (P < d->num_experts ? P : d->num_experts) + 15;
    if (PP * (d->hidden > d->inter ? d->hidden : d->inter) >= ((int64_t)1 << 30))
      return fail(QTIP_ERR_INVALID_ARG, "padded pairs * max(hidden, inter) must be below 2^30");
  }
  if ((int64_t)d->num_experts * d->hidden >= ((int64_t)1 << 31))
    return fail(QTIP_ERR_INVALID_ARG, "num_experts * hidden (the router weight) must be below 2^31 elements");
  if (d->arm_override != QTIP_ARM_AUTO && d->arm_override != QTIP_ARM_GEMV && d->arm_override != QTIP_ARM_GROUPED &&
      d->arm_override != QTIP_ARM_DEQUANT)
    return fail(QTIP_ERR_INVALID_ARG, "unknown arm_override");
  if (d->act_layout != QTIP_ACT_AUTO && d->act_layout != QTIP_ACT_ROWS && d->act_layout != QTIP_ACT_FRAGMENTS)
    return fail(QTIP_ERR_INVALID_ARG, "unknown act_layout");
  if (d->dequant_traffic_ratio < 0 || d->dequant_traffic_ratio > 1024)
    return fail(QTIP_ERR_INVALID_ARG, "dequant_traffic_ratio must be in [0, 1024]");
  if (d->out_dtype != QTIP_OUT_BF16 && d->out_dtype != QTIP_OUT_F32) return fail(QTIP_ERR_INVALID_ARG, "unknown out_dtype");
  const int32_t tm = d->tile_m == 0 ? QTIP_DEFAULT_TILE_M : d->tile_m;
  if (tm != 16 && tm != 32 && tm != 64) return fail(QTIP_ERR_INVALID_ARG, "tile_m must be 0, 16, 32 or 64");
  if (d->dispatch_tile_m < 0 || d->dispatch_tile_m > 1024)
    return fail(QTIP_ERR_INVALID_ARG, "dispatch_tile_m must be in [0, 1024]");
  if (d->decode_floor < 0 || d->decode_floor > 1024)
    return fail(QTIP_ERR_INVALID_ARG, "decode_floor must be in [0, 1024]");
  if (d->rung != QTIP_RUNG_BITSHIFT && d->rung != QTIP_RUNG_LUT)
    return fail(QTIP_ERR_INVALID_ARG, "rung must be QTIP_RUNG_BITSHIFT or QTIP_RUNG_LUT");
  if (d->small_batch != QTIP_SMALL_BATCH_FUSED && d->small_batch != QTIP_SMALL_BATCH_SEPARATE)
    return fail(QTIP_ERR_INVALID_ARG, "small_batch must be QTIP_SMALL_BATCH_FUSED or QTIP_SMALL_BATCH_SEPARATE");
  *tile_m = tm;
  return QTIP_OK;
}

// What a forward of n tokens uses: its kernel arm, and whether the grouped arm runs on the
// fragment-order activations (h, and x packed by an extra pass).
struct CallChoice {
  int32_t arm;
  int karm;
  bool frag, pack;
  bool route_in_gate_up;  // the batch is routed and binned inside the gate/up launch (SmallRoute)
};

CallChoice call_choice(const qtip_moe_plan_s* plan, int32_t n_tokens) {
  const qtip_moe_desc& d = plan->d;
  CallChoice c{};
  c.arm = d.arm_override != QTIP_ARM_AUTO
              ? d.arm_override
              : fill_select_arm(n_tokens, d.top_k, d.num_experts, plan->dispatch_tile_m, plan->dequant_ratio,
                                plan->decode_floor);
  c.karm = kernel_arm(c.arm);
  const double ppe = fill_pairs_per_woken_expert(n_tokens, d.top_k, d.num_experts);
  c.frag = plan->frag && c.karm == kArmGrouped && (d.act_layout == QTIP_ACT_FRAGMENTS || ppe >= kFragMinPairs);
  c.pack = c.frag && plan->pack && (d.act_layout == QTIP_ACT_FRAGMENTS || ppe >= kPackMinPairs);
  c.route_in_gate_up = d.small_batch == QTIP_SMALL_BATCH_FUSED && c.karm == kArmGemv && !c.frag &&
                       n_tokens <= kFusedRouteMaxTokens && (int64_t)n_tokens * d.top_k <= kSmallRouteMaxPairs;
  return c;
}

// The kernel configurations of a forward's two passes, and the down pass's token tasks
// (TokenCombine) where they apply: small batches routed inside the gate/up launch whose token
// tasks fit in one round on the CUs (measured on the V4 layer: one token; every further round
// adds a barrier and the first wave's serial sum, and with two tokens the launch of the combine
// kernel is already cheaper), a down configuration that can split a task's inputs over waves (by
// default one that can: 16 waves of 16-row tasks), and k x S waves within its workgroup, S the
// largest power of two that cuts the inputs into runs of at least two blocks.
constexpr long kTokenTaskRound = 256;  // CUs of an MI355X (gfx950)

struct PassPlan {
  int kv_gu, kv_dn;
  int tok_split;  // the token tasks' waves per pair, or 0: no token tasks (the combine kernel runs)
};

PassPlan pass_plan(const qtip_moe_plan_s* plan, const CallChoice& c, int32_t n_tokens) {
  const qtip_moe_desc& d = plan->d;
  PassPlan pp{};
  pp.kv_gu = fit_variant(resolve_variant(plan, c.karm, kModeGateUp, n_tokens), c.karm, d.inter);
  pp.kv_dn = fit_variant(resolve_variant(plan, c.karm, kModeSingle, n_tokens), c.karm, d.hidden);
  if (!c.route_in_gate_up) return pp;
  int kv = pp.kv_dn;
  VariantInfo v{};
  variant_info(kv, kArmGemv, v);
  if (!v.input_split && d.variant == kVariantDefault) {
    kv = fit_variant(1, kArmGemv, d.hidden);
    variant_info(kv, kArmGemv, v);
  }
  const int k = d.top_k, kblocks = d.inter / kKBlock;
  if (!v.input_split || k > v.waves || (long)n_tokens * (d.hidden / v.rows_per_task) > kTokenTaskRound) return pp;
  int S = 1;
  while (k * 2 * S <= v.waves && kblocks % (2 * S) == 0 && kblocks / (2 * S) >= 2) S *= 2;
  pp.kv_dn = kv;
  pp.tok_split = S;
  return pp;
}

// Scratch of a forward laid out for its own n tokens: only the buffers that call uses.
WsLayout call_layout(const qtip_moe_plan_s* plan, int32_t n_tokens) {
  const CallChoice c = call_choice(plan, n_tokens);
  return ws_layout(plan->d, plan->tile_m, n_tokens, c.karm == kArmDense, c.frag, c.pack);
}

// --- the allocation-free entry point's scratch ---------------------------------------------
// One array per GPU, held until the process ends.  Host code never uses the array's name as a
// device address (on the host it names a stand-in): the address of each device's copy comes
// from hipGetSymbolAddress, taken once per device with that device current, and only that
// address is passed to kernels.
constexpr size_t kScratchBytes = QTIP_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<char*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

qtip_status scratch_on(int dev, char** out) {
  char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      void* addr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!addr || (reinterpret_cast<uintptr_t>(addr) & 255))
        return fail(QTIP_ERR_HIP, "scratch symbol address is NULL or not 256-byte aligned");
      p = static_cast<char*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return QTIP_OK;
}

}  // namespace

extern "C" {

const char* qtip_status_string(qtip_status s) {
  switch (s) {
    case QTIP_OK: return "QTIP_OK";
    case QTIP_ERR_INVALID_ARG: return "QTIP_ERR_INVALID_ARG";
    case QTIP_ERR_INVALID_CONFIG: return "QTIP_ERR_INVALID_CONFIG";
    case QTIP_ERR_NOT_SUPPORTED: return "QTIP_ERR_NOT_SUPPORTED";
    case QTIP_ERR_HIP: return "QTIP_ERR_HIP";
    case QTIP_ERR_CAPTURING: return "QTIP_ERR_CAPTURING";
  }
  return "QTIP_ERR_UNKNOWN";
}

const char* qtip_last_error_detail(void) { return g_detail.c_str(); }

double qtip_fill_woken_experts(int32_t n, int32_t k, int32_t E) {
  if (!fill_args_ok(n, k, E, 1)) return -1.0;
  return fill_woken_experts(n, k, E);
}

double qtip_fill_pairs_per_woken_expert(int32_t n, int32_t k, int32_t E) {
  if (!fill_args_ok(n, k, E, 1)) return -1.0;
  return fill_pairs_per_woken_expert(n, k, E);
}

int32_t qtip_fill_select_grouped(int32_t n, int32_t k, int32_t E, int32_t tile_m) {
  if (!fill_args_ok(n, k, E, tile_m)) return -1;
  return fill_select_grouped(n, k, E, tile_m) ? 1 : 0;
}

int32_t qtip_fill_min_tokens(int32_t k, int32_t E, int32_t tile_m) {
  if (!fill_args_ok(1, k, E, tile_m)) return -1;
  return fill_min_tokens(k, E, tile_m);
}

qtip_status qtip_moe_plan_for_arch(const qtip_moe_desc* desc, const char* gcn_arch_name, qtip_moe_plan_t* out) {
  g_detail.clear();
  if (!out) return fail(QTIP_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int32_t tm = 0;
  qtip_status s = validate_desc(desc, &tm);
  if (s != QTIP_OK) return s;
  if (!arch_is_supported(gcn_arch_name))
    return fail(QTIP_ERR_NOT_SUPPORTED, std::string("arch '") + (gcn_arch_name ? gcn_arch_name : "(null)") +
                                            "' is not supported; this library carries gfx950 code only");
  int32_t variant = desc->variant;
  if (variant < 0 || variant >= kVariantCount) {
    std::fprintf(stderr, "qtip_moe: unknown kernel variant %d; keeping the default (0)\n", desc->variant);
    variant = 0;
  }
  auto* p = new (std::nothrow) qtip_moe_plan_s{};
  if (!p) return fail(QTIP_ERR_INVALID_ARG, "out of host memory");
  p->d = *desc;
  p->d.variant = variant;
  p->d.tile_m = tm;
  p->tile_m = tm;
  p->dispatch_tile_m = desc->dispatch_tile_m == 0 ? QTIP_DEFAULT_DISPATCH_TILE_M : desc->dispatch_tile_m;
  p->d.dispatch_tile_m = p->dispatch_tile_m;
  p->device = -1;
  p->decode_floor = desc->decode_floor != 0 ? desc->decode_floor
                    : (desc->rung == QTIP_RUNG_LUT ? QTIP_DEFAULT_DECODE_FLOOR_LUT : QTIP_DEFAULT_DECODE_FLOOR_BITSHIFT);
  p->d.decode_floor = p->decode_floor;
  p->min_tokens_grouped = fill_min_tokens(desc->top_k, desc->num_experts, p->dispatch_tile_m, p->decode_floor);
  p->dequant_ratio = desc->dequant_traffic_ratio == 0 ? kDequantTrafficRatio : desc->dequant_traffic_ratio;
  p->d.dequant_traffic_ratio = p->dequant_ratio;
  // Pairs per woken expert never decrease with n, so the automatic dispatch's dequantize
  // tokens form one interval: from the first n past the floor whose fill reaches the traffic
  // ratio up to the grouped arm's first n.
  p->dequant_lo = p->dequant_hi = 0;
  if (p->dequant_ratio < p->dispatch_tile_m) {
    const int32_t lo = fill_min_tokens(desc->top_k, desc->num_experts, p->dequant_ratio, p->decode_floor);
    int32_t hi = p->min_tokens_grouped;
    if (hi < 0 || hi > desc->max_tokens + 1) hi = desc->max_tokens + 1;
    if (lo > 0 && lo < hi) {
      p->dequant_lo = lo;
      p->dequant_hi = hi;
    }
  }
  p->dense = desc->arm_override == QTIP_ARM_DEQUANT ||
             (desc->arm_override == QTIP_ARM_AUTO && p->dequant_lo < p->dequant_hi);
  if (p->dense && (int64_t)desc->hidden * desc->inter >= ((int64_t)1 << 31)) {
    delete p;
    return fail(QTIP_ERR_INVALID_ARG, "the dequantize arm needs hidden * inter below 2^31 elements");
  }
  // Pairs per woken expert never decrease with n, so the fragment layout and the packing are
  // possible for some n <= max_tokens exactly when they are at max_tokens.
  const bool grouped_ok = desc->arm_override == QTIP_ARM_AUTO || desc->arm_override == QTIP_ARM_GROUPED;
  const double ppe_max = fill_pairs_per_woken_expert(desc->max_tokens, desc->top_k, desc->num_experts);
  p->frag = grouped_ok && desc->act_layout != QTIP_ACT_ROWS &&
            (desc->act_layout == QTIP_ACT_FRAGMENTS || ppe_max >= kFragMinPairs);
  p->pack = p->frag && (desc->act_layout == QTIP_ACT_FRAGMENTS || ppe_max >= kPackMinPairs);
  p->ws_bytes = ws_layout(p->d, tm, desc->max_tokens, p->dense, p->frag, p->pack).total;
  *out = p;
  return QTIP_OK;
}

qtip_status qtip_moe_plan(const qtip_moe_desc* desc, int device, qtip_moe_plan_t* out) {
  g_detail.clear();
  if (!out) return fail(QTIP_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int32_t tm = 0;
  qtip_status s = validate_desc(desc, &tm);
  if (s != QTIP_OK) return s;
  if (device < 0 || device >= kMaxDevices) return fail(QTIP_ERR_INVALID_ARG, "device index out of range");
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  s = qtip_moe_plan_for_arch(desc, prop.gcnArchName, out);
  if (s == QTIP_OK) (*out)->device = device;
  return s;
}

qtip_status qtip_moe_plan_destroy(qtip_moe_plan_t plan) {
  if (plan) prof_free(plan);
  delete plan;
  return QTIP_OK;
}

qtip_status qtip_moe_plan_info(qtip_moe_plan_t plan, int32_t* tile_m, size_t* workspace_bytes,
                               int32_t* min_tokens_grouped) {
  if (!plan) return fail(QTIP_ERR_INVALID_ARG, "plan is NULL");
  if (tile_m) *tile_m = plan->tile_m;
  if (workspace_bytes) *workspace_bytes = plan->ws_bytes;
  if (min_tokens_grouped) *min_tokens_grouped = plan->min_tokens_grouped;
  return QTIP_OK;
}

static void shape_of(int kv, int karm, qtip_moe_kernel_shape* out) {
  VariantInfo v{};
  variant_info(kv, karm, v);
  out->variant = kv;
  out->waves_per_workgroup = v.waves;
  out->rows_per_task = v.rows_per_task;
  out->pairs_per_decode = v.pairs_per_decode;
}

qtip_status qtip_moe_plan_schedule(qtip_moe_plan_t plan, int32_t n_tokens, qtip_moe_schedule* out) {
  if (!plan || !out) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  if (n_tokens < 1) return fail(QTIP_ERR_INVALID_CONFIG, "n_tokens must be >= 1");
  const int32_t arm = qtip_moe_select_arm(plan, n_tokens);
  const int karm = kernel_arm(arm);
  out->arm = arm;
  out->tile_m = plan->tile_m;
  const CallChoice c = call_choice(plan, n_tokens);
  const PassPlan pp = pass_plan(plan, c, n_tokens);
  out->route_in_gate_up = c.route_in_gate_up ? 1 : 0;
  out->combine_in_down = pp.tok_split > 0 ? 1 : 0;
  shape_of(pp.kv_gu, karm, &out->gate_up);
  shape_of(pp.kv_dn, karm, &out->down);
  return QTIP_OK;
}

int32_t qtip_moe_select_grouped(qtip_moe_plan_t plan, int32_t n_tokens) {
  if (!plan || n_tokens < 1) return -1;
  return fill_select_grouped(n_tokens, plan->d.top_k, plan->d.num_experts, plan->dispatch_tile_m, plan->decode_floor)
             ? 1 : 0;
}

int32_t qtip_moe_select_arm(qtip_moe_plan_t plan, int32_t n_tokens) {
  if (!plan || n_tokens < 1) return -1;
  if (plan->d.arm_override != QTIP_ARM_AUTO) return plan->d.arm_override;
  return fill_select_arm(n_tokens, plan->d.top_k, plan->d.num_experts, plan->dispatch_tile_m, plan->dequant_ratio,
                         plan->decode_floor);
}

qtip_status qtip_arch_witness(int device, void* stream) {
  g_detail.clear();
  if (device < 0 || device >= kMaxDevices) return fail(QTIP_ERR_INVALID_ARG, "device index out of range");
  int cur = 0;
  qtip_status s = current_device(&cur);
  if (s != QTIP_OK) return s;
  if (cur != device) {
    hipError_t e = hipSetDevice(device);
    if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  }
  s = witness_on(device, (hipStream_t)stream);
  if (cur != device) (void)hipSetDevice(cur);
  return s;
}

qtip_status qtip_moe_route(qtip_moe_plan_t plan, const float* logits, int32_t n_tokens, int32_t* topk_idx,
                           float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                           int32_t* tile_map, int32_t* n_tiles, void* stream) {
  g_detail.clear();
  if (!plan || !logits || !topk_idx || !topk_w || !counts || !offsets || !sorted_pair || !tile_map || !n_tiles)
    return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  if (n_tokens <= 0 || n_tokens > plan->d.max_tokens)
    return fail(QTIP_ERR_INVALID_CONFIG, "n_tokens must be in [1, max_tokens]");
  const hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  qtip_status s = ensure_device(plan, st, &dev);
  if (s != QTIP_OK) return s;
  const qtip_moe_desc& d = plan->d;
  hipError_t e;
  if (n_tokens <= kFusedRouteMaxTokens) {  // the same kernels as the forward's routing
    e = launch_route_bin(logits, 1, n_tokens, d.num_experts, d.top_k, topk_idx, topk_w, plan->tile_m, counts, offsets,
                         sorted_pair, tile_map, n_tiles, nullptr, nullptr, nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "route/bin launch");
    plan->stats.route_launches++;
    return QTIP_OK;
  }
  e = launch_route_topk(logits, 1, n_tokens, d.num_experts, d.top_k, topk_idx, topk_w, st);
  if (e != hipSuccess) return hip_fail(e, "route_topk launch");
  plan->stats.route_launches++;
  e = launch_bin(topk_idx, n_tokens * d.top_k, d.num_experts, plan->tile_m, counts, offsets, sorted_pair, tile_map,
                 n_tiles, nullptr, nullptr, nullptr, st);
  if (e != hipSuccess) return hip_fail(e, "bin launch");
  plan->stats.route_launches++;
  return QTIP_OK;
}

qtip_status qtip_expert_matmul(qtip_moe_plan_t plan, int32_t arm, const uint8_t* codes, const uint16_t* scales,
                               const uint16_t* lut, int32_t num_experts, int32_t rows, int32_t cols,
                               const void* a_bf16, int32_t n_rows_a, const int32_t* unit_map, int32_t n_units,
                               float* y, void* stream) {
  g_detail.clear();
  if (!plan || !codes || !scales || !lut || !a_bf16 || !unit_map || !y) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  if (arm != QTIP_ARM_GEMV && arm != QTIP_ARM_GROUPED) return fail(QTIP_ERR_INVALID_ARG, "arm must be GEMV or GROUPED");
  if (num_experts < 1 || rows < 16 || rows % 16 || cols < kKBlock || cols % kKBlock || n_rows_a < 1)
    return fail(QTIP_ERR_INVALID_ARG, "bad shape: rows % 16, cols % 128, num_experts >= 1, n_rows_a >= 1");
  if ((reinterpret_cast<uintptr_t>(lut) & 15) || (reinterpret_cast<uintptr_t>(a_bf16) & 15) ||
      (reinterpret_cast<uintptr_t>(codes) & 7))
    return fail(QTIP_ERR_INVALID_ARG, "lut and a_bf16 must be 16-byte aligned, codes 8-byte aligned");
  if (n_units <= 0) return fail(QTIP_ERR_INVALID_CONFIG, "n_units must be >= 1 (an empty launch is an error)");
  if ((int64_t)n_rows_a * cols >= ((int64_t)1 << 30) || (int64_t)rows * (cols / 4) >= ((int64_t)1 << 31))
    return fail(QTIP_ERR_INVALID_ARG, "n_rows_a * cols must be below 2^30 and rows * cols / 4 below 2^31");
  const hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  qtip_status s = ensure_device(plan, st, &dev);
  if (s != QTIP_OK) return s;
  const int karm = arm == QTIP_ARM_GROUPED ? kArmGrouped : kArmGemv;
  const int kv = fit_variant(resolve_variant(plan, karm, kModeSingle, 0), karm, rows);
  VariantInfo vi{};
  variant_info(kv, karm, vi);
  ExpertParams p{};
  p.codes0 = codes;
  p.scale0 = scales;
  p.lut = lut;
  p.act = reinterpret_cast<const uint16_t*>(a_bf16);
  p.act_row_div = 1;
  p.units = unit_map;
  p.n_units_host = n_units;
  p.num_experts = num_experts;
  p.rows = rows;
  p.cols = cols;
  p.n_pos = n_rows_a;
  p.n_act_rows = n_rows_a;
  p.out = y;
  p.n_out_rows = n_rows_a;
  p.n_xcd = xcd_count(dev);
  const LaunchShape shape =
      persistent_shape(dev, (size_t)n_units * (rows / vi.rows_per_task), vi.waves, karm == kArmGemv);
  hipError_t e = launch_expert(kModeSingle, karm, kv, plan->d.rung, p, shape.grid, shape.waves, st);
  if (e != hipSuccess) return hip_fail(e, "expert kernel launch");
  if (arm == QTIP_ARM_GROUPED) {
    plan->stats.grouped_launches++;
    plan->stats.grouped_variant_launches[kv]++;
  } else {
    plan->stats.gemv_launches++;
    plan->stats.gemv_variant_launches[kv]++;
  }
  return QTIP_OK;
}

}  // extern "C"

namespace {

// The layer from router logits (logits != NULL) or from hidden states through the router
// GEMM (w_router != NULL; its K-chunk partial sums go to the workspace and the top-k kernel
// adds them).  The workspace regions are laid out for the plan's max_tokens, or, with
// layout_for_n (the allocation-free entry point), for this call's n_tokens only.
qtip_status forward_impl(qtip_moe_plan_t plan, const qtip_moe_weights* w, const void* x_bf16, const float* logits,
                         const void* w_router, int32_t n_tokens, void* out, void* workspace, size_t workspace_bytes,
                         void* stream, bool layout_for_n = false) {
  g_detail.clear();
  if (!plan || !w || !x_bf16 || !(logits || w_router) || !out || !workspace)
    return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  if (reinterpret_cast<uintptr_t>(w_router) & 15) return fail(QTIP_ERR_INVALID_ARG, "w_router must be 16-byte aligned");
  if (!w->codes_gate || !w->codes_up || !w->codes_down || !w->scale_gate || !w->scale_up || !w->scale_down || !w->lut)
    return fail(QTIP_ERR_INVALID_ARG, "NULL weight pointer");
  if ((reinterpret_cast<uintptr_t>(w->lut) & 15) || (reinterpret_cast<uintptr_t>(x_bf16) & 15) ||
      (reinterpret_cast<uintptr_t>(out) & 15) || (reinterpret_cast<uintptr_t>(w->codes_gate) & 7) ||
      (reinterpret_cast<uintptr_t>(w->codes_up) & 7) || (reinterpret_cast<uintptr_t>(w->codes_down) & 7))
    return fail(QTIP_ERR_INVALID_ARG, "lut, x and out must be 16-byte aligned, codes 8-byte aligned");
  if (n_tokens <= 0 || n_tokens > plan->d.max_tokens)
    return fail(QTIP_ERR_INVALID_CONFIG, "n_tokens must be in [1, max_tokens] (an empty launch is an error)");
  const size_t ws_need = layout_for_n ? call_layout(plan, n_tokens).total : plan->ws_bytes;
  if (workspace_bytes < ws_need || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(QTIP_ERR_INVALID_ARG, "workspace too small or not 256-byte aligned");
  const hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  qtip_status s = ensure_device(plan, st, &dev);
  if (s != QTIP_OK) return s;

  const qtip_moe_desc& d = plan->d;
  const CallChoice choice = call_choice(plan, n_tokens);
  const int32_t arm = choice.arm;
  const int karm = choice.karm;
  if (karm == kArmDense && !plan->dense) return fail(QTIP_ERR_INVALID_CONFIG, "the plan has no dequantize workspace");
  const WsLayout L = layout_for_n ? call_layout(plan, n_tokens)
                                  : ws_layout(d, plan->tile_m, d.max_tokens, plan->dense, plan->frag, plan->pack);
  char* ws = reinterpret_cast<char*>(workspace);
  int32_t* topk_idx = reinterpret_cast<int32_t*>(ws + L.topk_idx);
  float* topk_w = reinterpret_cast<float*>(ws + L.topk_w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted_pair = reinterpret_cast<int32_t*>(ws + L.sorted_pair);
  int32_t* tile_map = reinterpret_cast<int32_t*>(ws + L.tile_map);
  int32_t* pair_pos = reinterpret_cast<int32_t*>(ws + L.pair_pos);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(ws + L.n_tiles);
  int32_t* unit_map = reinterpret_cast<int32_t*>(ws + L.unit_map);
  int32_t* n_units = reinterpret_cast<int32_t*>(ws + L.n_units);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  float* y = reinterpret_cast<float*>(ws + L.y);
  const int32_t P = n_tokens * d.top_k;

  hipError_t e = prof_mark(plan, 0, st);
  if (e != hipSuccess) return hip_fail(e, "profile event");
  const float* lg = logits;
  int32_t n_part = 1;
  if (w_router) {
    n_part = router_split(n_tokens, d.num_experts, d.hidden);
    float* part = reinterpret_cast<float*>(ws + L.router_part);
    e = launch_router_gemm(reinterpret_cast<const uint16_t*>(x_bf16), reinterpret_cast<const uint16_t*>(w_router),
                           n_tokens, d.num_experts, d.hidden, n_part, xcd_count(dev), part, st);
    if (e != hipSuccess) return hip_fail(e, "router GEMM launch");
    plan->stats.router_launches++;
    lg = part;
  }
  // The grouped arm's activation layout: fragment order over padded positions for h (and the
  // down pass) from kFragMinPairs pairs per woken expert, for x too (an extra packing pass)
  // from kPackMinPairs; gathered rows below.
  const bool frag = choice.frag;
  int32_t* padded_pair = reinterpret_cast<int32_t*>(ws + L.padded_pair);
  int32_t* n_pad = reinterpret_cast<int32_t*>(ws + L.n_pad);
  uint16_t* xs = reinterpret_cast<uint16_t*>(ws + L.xs);
  const int32_t pp_max = (int32_t)pad_positions(d, n_tokens);
  // kernel configurations of the two passes; each pass gets its own decode units (runs of its
  // pairs per decode), so every task of a pass is one decode of its rows
  const PassPlan pp = pass_plan(plan, choice, n_tokens);
  const int kv_gu = pp.kv_gu, kv_dn = pp.kv_dn;
  VariantInfo vi_gu{}, vi_dn{};
  variant_info(kv_gu, karm, vi_gu);
  variant_info(kv_dn, karm, vi_dn);
  UnitMaps um{};
  um.unit_pairs[0] = vi_gu.pairs_per_decode;
  um.unit_pairs[1] = vi_dn.pairs_per_decode;
  um.map[0] = unit_map;
  um.map[1] = unit_map + 3 * L.max_units;
  um.count[0] = n_units;
  um.count[1] = n_units + 1;
  um.pad[0] = frag ? reinterpret_cast<int32_t*>(ws + L.unit_pad) : nullptr;
  um.pad[1] = frag ? reinterpret_cast<int32_t*>(ws + L.unit_pad) + L.max_units : nullptr;
  const bool spread = karm == kArmGemv;
  const LaunchShape shape_gu =
      persistent_shape(dev, max_units_for(d, n_tokens, vi_gu.pairs_per_decode) * (d.inter / vi_gu.rows_per_task),
                       vi_gu.waves, spread, vi_gu.input_split, d.hidden / kKBlock);
  LaunchShape shape_dn =
      persistent_shape(dev, max_units_for(d, n_tokens, vi_dn.pairs_per_decode) * (d.hidden / vi_dn.rows_per_task),
                       vi_dn.waves, spread, vi_dn.input_split, d.inter / kKBlock);
  if (pp.tok_split) {
    // token tasks: one workgroup of k x S waves per token and row block, persistent over the CUs
    const long tok_tasks = (long)n_tokens * (d.hidden / vi_dn.rows_per_task);
    const long cus = g_cu_count[dev].load(std::memory_order_acquire);
    shape_dn = LaunchShape{(int)(tok_tasks < cus ? tok_tasks : cus), d.top_k * pp.tok_split, pp.tok_split};
  }
  if (choice.route_in_gate_up) {
    // routed and binned inside the gate/up launch below (the "route" stage is empty)
    if ((e = prof_mark(plan, 1, st)) != hipSuccess) return hip_fail(e, "profile event");
  } else if (n_tokens <= kFusedRouteMaxTokens) {
    // one workgroup routes and bins a small batch (the "route" stage then holds both)
    e = launch_route_bin(lg, n_part, n_tokens, d.num_experts, d.top_k, topk_idx, topk_w, plan->tile_m, counts, offsets,
                         sorted_pair, tile_map, n_tiles, frag ? padded_pair : nullptr, frag ? n_pad : nullptr, &um, st);
    if (e != hipSuccess) return hip_fail(e, "route/bin launch");
    if ((e = prof_mark(plan, 1, st)) != hipSuccess) return hip_fail(e, "profile event");
    plan->stats.route_launches += 1;
  } else {
    e = launch_route_topk(lg, n_part, n_tokens, d.num_experts, d.top_k, topk_idx, topk_w, st);
    if (e != hipSuccess) return hip_fail(e, "route_topk launch");
    if ((e = prof_mark(plan, 1, st)) != hipSuccess) return hip_fail(e, "profile event");
    e = launch_bin(topk_idx, P, d.num_experts, plan->tile_m, counts, offsets, sorted_pair, tile_map, n_tiles,
                   frag ? padded_pair : nullptr, frag ? n_pad : nullptr, &um, st);
    if (e != hipSuccess) return hip_fail(e, "bin launch");
    plan->stats.route_launches += 2;
  }
  const bool pack = choice.pack;
  if (pack) {
    e = launch_pack_act(reinterpret_cast<const uint16_t*>(x_bf16), padded_pair, n_pad, d.top_k, d.hidden, pp_max, xs,
                        st);
    if (e != hipSuccess) return hip_fail(e, "activation pack launch");
  }
  if ((e = prof_mark(plan, 2, st)) != hipSuccess) return hip_fail(e, "profile event");

  uint16_t* dense_gate = reinterpret_cast<uint16_t*>(ws + L.dense_gate);
  uint16_t* dense_up = reinterpret_cast<uint16_t*>(ws + L.dense_up);
  uint16_t* dense_down = reinterpret_cast<uint16_t*>(ws + L.dense_down);
  if (karm == kArmDense) {
    // materialise the woken experts' three matrices (counts from the binning just launched)
    DequantParams q{};
    q.codes0 = w->codes_gate;
    q.codes1 = w->codes_up;
    q.lut = w->lut;
    q.counts = counts;
    q.num_experts = d.num_experts;
    q.rows = d.inter;
    q.cols = d.hidden;
    q.expert = -1;
    q.out0 = dense_gate;
    q.out1 = dense_up;
    q.out_expert_stride = (int64_t)d.inter * d.hidden;
    q.fragment_order = 1;
    e = launch_dequant(q, plan->d.rung, persistent_grid(dev, (size_t)d.num_experts * (d.inter / 16), kDequantWaves), st);
    if (e != hipSuccess) return hip_fail(e, "dequantize launch");
    q.codes0 = w->codes_down;
    q.codes1 = nullptr;
    q.rows = d.hidden;
    q.cols = d.inter;
    q.out0 = dense_down;
    q.out1 = nullptr;
    e = launch_dequant(q, plan->d.rung, persistent_grid(dev, (size_t)d.num_experts * (d.hidden / 16), kDequantWaves), st);
    if (e != hipSuccess) return hip_fail(e, "dequantize launch");
    plan->stats.dequant_launches += 2;
  }

  ExpertParams gu{};
  gu.dense0 = dense_gate;
  gu.dense1 = dense_up;
  gu.dense_counts = counts;
  gu.codes0 = w->codes_gate;
  gu.codes1 = w->codes_up;
  gu.scale0 = w->scale_gate;
  gu.scale1 = w->scale_up;
  gu.lut = w->lut;
  gu.act = reinterpret_cast<const uint16_t*>(x_bf16);
  gu.act_row_map = sorted_pair;
  gu.act_row_div = d.top_k;
  gu.units = um.map[0];
  gu.n_units_dev = um.count[0];
  gu.num_experts = d.num_experts;
  gu.rows = d.inter;
  gu.cols = d.hidden;
  gu.n_pos = P;
  gu.n_act_rows = n_tokens;
  gu.out = h;
  gu.n_out_rows = P;
  gu.n_xcd = xcd_count(dev);
  if (frag) {
    gu.unit_pad = um.pad[0];
    gu.n_pad_max = pp_max;
  }
  if (pack) {
    gu.act = xs;
    gu.act_frag = 1;
  }
  gu.ksplit = shape_gu.ksplit;
  if (choice.route_in_gate_up) {
    SmallRoute& r = gu.route;
    r.logits = lg;
    r.n_part = n_part;
    r.n = n_tokens;
    r.top_k = d.top_k;
    r.topk_idx = topk_idx;
    r.topk_w = topk_w;
    r.sorted_pair = sorted_pair;
    r.pair_pos = pp.tok_split ? pair_pos : nullptr;
    for (int i = 0; i < 2; ++i) {
      r.unit_pairs[i] = um.unit_pairs[i];
      r.units[i] = um.map[i];
      r.n_units[i] = um.count[i];
    }
  }
  e = launch_expert(kModeGateUp, karm, kv_gu, plan->d.rung, gu, shape_gu.grid, shape_gu.waves, st);
  if (e != hipSuccess) return hip_fail(e, "gate/up expert kernel launch");
  if ((e = prof_mark(plan, 3, st)) != hipSuccess) return hip_fail(e, "profile event");

  ExpertParams dn{};
  dn.dense0 = dense_down;
  dn.dense_counts = counts;
  dn.codes0 = w->codes_down;
  dn.scale0 = w->scale_down;
  dn.lut = w->lut;
  dn.act = h;
  dn.act_row_div = 1;
  dn.units = um.map[1];
  dn.n_units_dev = um.count[1];
  dn.num_experts = d.num_experts;
  dn.rows = d.hidden;
  dn.cols = d.inter;
  dn.n_pos = P;
  dn.n_act_rows = P;
  dn.out = y;
  dn.out_row_map = sorted_pair;
  dn.n_out_rows = P;
  dn.n_xcd = xcd_count(dev);
  if (frag) {
    dn.unit_pad = um.pad[1];
    dn.act_frag = 1;
    dn.n_pad_max = pp_max;
  }
  dn.ksplit = shape_dn.ksplit;
  if (pp.tok_split) {
    // the down pass adds each token's pairs into out; pair p's h row is its binned position
    dn.tok = TokenCombine{topk_idx, topk_w, pair_pos, out, n_tokens, d.top_k, d.out_dtype == QTIP_OUT_BF16 ? 1 : 0};
  }
  e = launch_expert(kModeSingle, karm, kv_dn, plan->d.rung, dn, shape_dn.grid, shape_dn.waves, st);
  if (e != hipSuccess) return hip_fail(e, "down expert kernel launch");
  if ((e = prof_mark(plan, 4, st)) != hipSuccess) return hip_fail(e, "profile event");
  if (karm == kArmGrouped) {
    plan->stats.grouped_launches += 2;
    plan->stats.grouped_variant_launches[kv_gu]++;
    plan->stats.grouped_variant_launches[kv_dn]++;
  } else if (karm == kArmDense) {
    plan->stats.dequant_launches += 2;
  } else {
    plan->stats.gemv_launches += 2;
    plan->stats.gemv_variant_launches[kv_gu]++;
    plan->stats.gemv_variant_launches[kv_dn]++;
  }

  if (pp.tok_split) {
    plan->stats.combined_in_down++;  // the "combine" stage is empty
  } else {
    e = launch_combine(y, topk_w, n_tokens, d.top_k, d.hidden, out, d.out_dtype == QTIP_OUT_BF16, st);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    plan->stats.combine_launches++;
  }
  if ((e = prof_mark(plan, 5, st)) != hipSuccess) return hip_fail(e, "profile event");
  if (plan->prof_capacity) plan->prof_recorded++;
  if (choice.route_in_gate_up) plan->stats.routed_in_gate_up++;
  plan->stats.forward_calls++;
  plan->stats.last_arm = arm;
  plan->stats.last_n_tokens = n_tokens;
  return QTIP_OK;
}

}  // namespace

extern "C" {

qtip_status qtip_moe_forward(qtip_moe_plan_t plan, const qtip_moe_weights* w, const void* x_bf16, const float* logits,
                             int32_t n_tokens, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits) {
    g_detail.clear();
    return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  }
  return forward_impl(plan, w, x_bf16, logits, nullptr, n_tokens, out, workspace, workspace_bytes, stream);
}

qtip_status qtip_moe_forward_hidden(qtip_moe_plan_t plan, const qtip_moe_weights* w, const void* w_router_bf16,
                                    const void* x_bf16, int32_t n_tokens, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!w_router_bf16) {
    g_detail.clear();
    return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  }
  return forward_impl(plan, w, x_bf16, nullptr, w_router_bf16, n_tokens, out, workspace, workspace_bytes, stream);
}

qtip_status qtip_moe_forward_noalloc(qtip_moe_plan_t plan, const qtip_moe_weights* w, const void* x_bf16,
                                     const float* logits, int32_t n_tokens, void* out, void* stream) {
  g_detail.clear();
  if (!plan || !logits) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  if (n_tokens <= 0 || n_tokens > plan->d.max_tokens)
    return fail(QTIP_ERR_INVALID_CONFIG, "n_tokens must be in [1, max_tokens] (an empty launch is an error)");
  // the size check needs host scalars only, so an oversized call touches no device state
  const size_t need = call_layout(plan, n_tokens).total;
  if (need > kScratchBytes)
    return fail(QTIP_ERR_INVALID_CONFIG, "this layer needs " + std::to_string(need) +
                                             " bytes of scratch for " + std::to_string(n_tokens) +
                                             " tokens; the allocation-free entry point holds " +
                                             std::to_string(kScratchBytes) + " (QTIP_NOALLOC_SCRATCH_BYTES)");
  int dev = 0;
  qtip_status s = current_device(&dev);
  if (s != QTIP_OK) return s;
  char* ptr = nullptr;
  if ((s = scratch_on(dev, &ptr)) != QTIP_OK) return s;
  return forward_impl(plan, w, x_bf16, logits, nullptr, n_tokens, out, ptr, kScratchBytes, stream, true);
}

qtip_status qtip_moe_router_logits(qtip_moe_plan_t plan, const void* x_bf16, const void* w_router_bf16,
                                   int32_t n_tokens, float* logits, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  g_detail.clear();
  if (!plan || !x_bf16 || !w_router_bf16 || !logits || !workspace) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  if ((reinterpret_cast<uintptr_t>(x_bf16) & 15) || (reinterpret_cast<uintptr_t>(w_router_bf16) & 15))
    return fail(QTIP_ERR_INVALID_ARG, "x and w_router must be 16-byte aligned");
  if (n_tokens <= 0 || n_tokens > plan->d.max_tokens)
    return fail(QTIP_ERR_INVALID_CONFIG, "n_tokens must be in [1, max_tokens] (an empty launch is an error)");
  if (workspace_bytes < plan->ws_bytes || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(QTIP_ERR_INVALID_ARG, "workspace too small or not 256-byte aligned");
  const hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  qtip_status s = ensure_device(plan, st, &dev);
  if (s != QTIP_OK) return s;
  const qtip_moe_desc& d = plan->d;
  const int32_t S = router_split(n_tokens, d.num_experts, d.hidden);
  const WsLayout L = ws_layout(d, plan->tile_m, d.max_tokens, plan->dense, plan->frag, plan->pack);
  float* part = S == 1 ? logits : reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + L.router_part);
  hipError_t e = launch_router_gemm(reinterpret_cast<const uint16_t*>(x_bf16),
                                    reinterpret_cast<const uint16_t*>(w_router_bf16), n_tokens, d.num_experts,
                                    d.hidden, S, xcd_count(dev), part, st);
  if (e != hipSuccess) return hip_fail(e, "router GEMM launch");
  plan->stats.router_launches++;
  if (S > 1) {
    e = launch_router_reduce(part, S, (int64_t)n_tokens * d.num_experts, logits, st);
    if (e != hipSuccess) return hip_fail(e, "router reduce launch");
  }
  return QTIP_OK;
}

qtip_status qtip_moe_dequant_range(qtip_moe_plan_t plan, int32_t* n_lo, int32_t* n_hi) {
  g_detail.clear();
  if (!plan || !n_lo || !n_hi) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  *n_lo = plan->dequant_lo;
  *n_hi = plan->dequant_hi;
  return QTIP_OK;
}

int32_t qtip_fill_select_arm(int32_t n, int32_t k, int32_t E, int32_t tile_m, int32_t dequant_ratio) {
  if (!fill_args_ok(n, k, E, tile_m) || dequant_ratio < 1) return -1;
  return fill_select_arm(n, k, E, tile_m, dequant_ratio);
}

qtip_status qtip_moe_dequantize(qtip_moe_plan_t plan, const qtip_moe_weights* w, int32_t matrix, int32_t expert,
                                void* dense_out, void* stream) {
  g_detail.clear();
  if (!plan || !w || !dense_out || !w->lut) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  const qtip_moe_desc& d = plan->d;
  if (matrix < 0 || matrix > 2) return fail(QTIP_ERR_INVALID_ARG, "matrix must be 0 (gate), 1 (up) or 2 (down)");
  if (expert < 0 || expert >= d.num_experts) return fail(QTIP_ERR_INVALID_ARG, "expert out of range");
  const uint8_t* codes = matrix == 0 ? w->codes_gate : (matrix == 1 ? w->codes_up : w->codes_down);
  if (!codes) return fail(QTIP_ERR_INVALID_ARG, "NULL codes");
  if ((reinterpret_cast<uintptr_t>(codes) & 7) || (reinterpret_cast<uintptr_t>(w->lut) & 15) ||
      (reinterpret_cast<uintptr_t>(dense_out) & 15))
    return fail(QTIP_ERR_INVALID_ARG, "codes must be 8-byte aligned, lut and dense_out 16-byte aligned");
  const hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  qtip_status s = ensure_device(plan, st, &dev);
  if (s != QTIP_OK) return s;
  DequantParams q{};
  q.codes0 = codes;
  q.lut = w->lut;
  q.num_experts = d.num_experts;
  q.rows = matrix == 2 ? d.hidden : d.inter;
  q.cols = matrix == 2 ? d.inter : d.hidden;
  q.expert = expert;
  q.out0 = reinterpret_cast<uint16_t*>(dense_out);
  q.out_expert_stride = 0;
  q.fragment_order = 0;
  hipError_t e = launch_dequant(q, plan->d.rung, persistent_grid(dev, (size_t)(q.rows / 16), kDequantWaves), st);
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  plan->stats.dequant_launches++;
  return QTIP_OK;
}

int32_t qtip_moe_router_split(qtip_moe_plan_t plan, int32_t n_tokens) {
  if (!plan || n_tokens < 1) return -1;
  return router_split(n_tokens, plan->d.num_experts, plan->d.hidden);
}

qtip_status qtip_moe_profile_enable(qtip_moe_plan_t plan, int32_t capacity) {
  g_detail.clear();
  if (!plan) return fail(QTIP_ERR_INVALID_ARG, "plan is NULL");
  if (capacity < 0 || capacity > 4096) return fail(QTIP_ERR_INVALID_ARG, "capacity must be in [0, 4096]");
  prof_free(plan);
  if (capacity == 0) return QTIP_OK;
  plan->prof_events.assign((size_t)capacity * (kStages + 1), nullptr);
  for (auto& ev : plan->prof_events) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      prof_free(plan);
      return hip_fail(e, "hipEventCreate");
    }
  }
  plan->prof_capacity = capacity;
  return QTIP_OK;
}

qtip_status qtip_moe_profile_read(qtip_moe_plan_t plan, double* stage_ms, int32_t* n_forwards) {
  g_detail.clear();
  if (!plan || !stage_ms || !n_forwards) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  for (int b = 0; b < kStages; ++b) stage_ms[b] = 0.0;
  *n_forwards = 0;
  if (plan->prof_capacity == 0) return fail(QTIP_ERR_INVALID_CONFIG, "profiling is not enabled");
  const int64_t n = plan->prof_recorded < plan->prof_capacity ? plan->prof_recorded : plan->prof_capacity;
  for (int64_t slot = 0; slot < n; ++slot) {
    hipEvent_t* ev = &plan->prof_events[slot * (kStages + 1)];
    hipError_t e = hipEventSynchronize(ev[kStages]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    for (int b = 0; b < kStages; ++b) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, ev[b], ev[b + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      stage_ms[b] += ms;
    }
  }
  *n_forwards = (int32_t)n;
  plan->prof_recorded = 0;
  return QTIP_OK;
}

qtip_status qtip_measure_lut_gather(int32_t rounds, uint32_t* sink, size_t sink_elems, void* stream,
                                    double* lookups_per_second) {
  g_detail.clear();
  if (!sink || !lookups_per_second) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  if (rounds < 1 || rounds > (1 << 20)) return fail(QTIP_ERR_INVALID_CONFIG, "rounds must be in [1, 2^20]");
  const hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  qtip_status s = current_device(&dev);
  if (s != QTIP_OK) return s;
  if ((s = witness_on(dev, st)) != QTIP_OK) return s;
  const int grid = g_cu_count[dev].load(std::memory_order_acquire);
  if (sink_elems < (size_t)grid * 1024) return fail(QTIP_ERR_INVALID_ARG, "sink needs CU count x 1024 elements");
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipEventRecord(e0, st);
  if (e == hipSuccess) e = launch_gather_probe(grid, rounds, sink, st);
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_fail(e, "gather probe");
  *lookups_per_second = (double)grid * 1024.0 * 16.0 * rounds / (ms * 1e-3);
  return QTIP_OK;
}

qtip_status qtip_moe_stats(qtip_moe_plan_t plan, qtip_moe_stats_t* out) {
  if (!plan || !out) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  *out = plan->stats;
  return QTIP_OK;
}

qtip_status qtip_moe_stats_reset(qtip_moe_plan_t plan) {
  if (!plan) return fail(QTIP_ERR_INVALID_ARG, "plan is NULL");
  plan->stats = qtip_moe_stats_t{};
  return QTIP_OK;
}

qtip_status qtip_moe_engaged_line(qtip_moe_plan_t plan, int32_t n_tokens, char* buf, size_t buf_len) {
  if (!plan || !buf || buf_len == 0) return fail(QTIP_ERR_INVALID_ARG, "NULL argument");
  if (n_tokens < 1) return fail(QTIP_ERR_INVALID_CONFIG, "n_tokens must be >= 1");
  const qtip_moe_desc& d = plan->d;
  const int32_t arm = qtip_moe_select_arm(plan, n_tokens);
  const double ppe = fill_pairs_per_woken_expert(n_tokens, d.top_k, d.num_experts);
  std::snprintf(buf, buf_len,
                "qtip_moe: %s arm for %d tokens x top-%d of %d experts; mean m-tile fill %.1f%% "
                "(%.2f pairs per woken expert, tile_m=%d); dispatch threshold %d pairs, GEMV up to %d tokens, "
                "grouped from %d tokens%s",
                arm == QTIP_ARM_GROUPED ? "grouped" : (arm == QTIP_ARM_DEQUANT ? "dequantize" : "GEMV"), n_tokens,
                d.top_k, d.num_experts,
                100.0 * ppe / plan->tile_m, ppe, plan->tile_m, plan->dispatch_tile_m, plan->decode_floor,
                plan->min_tokens_grouped,
                d.arm_override != QTIP_ARM_AUTO ? " (arm pinned by the plan)" : "");
  return QTIP_OK;
}

qtip_status qtip_moe_log_engaged(qtip_moe_plan_t plan, int32_t n_tokens, int32_t* printed) {
  if (printed) *printed = 0;
  char line[512];
  const qtip_status s = qtip_moe_engaged_line(plan, n_tokens, line, sizeof(line));
  if (s != QTIP_OK) return s;
  const int32_t arm = qtip_moe_select_arm(plan, n_tokens);
  if (arm < 0 || arm > 3 || plan->engaged_logged[arm]) return QTIP_OK;
  plan->engaged_logged[arm] = true;
  std::fprintf(stderr, "%s\n", line);
  std::fflush(stderr);
  if (printed) *printed = 1;
  return QTIP_OK;
}

}  // extern "C"
