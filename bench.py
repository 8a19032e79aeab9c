#!/usr/bin/env python3
"""Benchmark of the trellis-quantized MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--curve NAMES]

A step is one qtip_moe_forward (route, bin, gate+up, down, combine) over one batch of the
workload, with weights and inputs already resident in HBM.  The headline workload is the
largest V4-shaped layer (E=256, top-6, hidden 4096, expert intermediate 2048, n=1024 tokens,
uniform routing, seed 0), in the plan a caller of that size uses (max_tokens = n, automatic arm
and kernel configuration, bf16 output).  Prints ONE JSON line: tokens/s over the timed steps,
the roofline of the dominant kernel (gate+up: packed-weight bytes per launch over its
HIP-event-measured duration, against 8 TB/s), the CPU oracle timed on a bounded sample over
the host's cores, and in "detail.curve" the same measurements for the other workloads (the
metric against token count n: V4 n = 1, 32, 128, 512, 683, Zipf(1.1) n = 256, and the tiny
layer).

Other modes (not used by the driver):
  --sweep PATH        both arms forced at n in {8,16,32,64,128,256,512,683,1024}; JSON lines to PATH
  --calibrate-copy    run one device copy of known size first (for scaling PMC byte counters)
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + packed-weight HBM GB/s (% peak) vs token count n"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
# VALU decode ceiling: 256 CUs x 64 lanes x 2.4 GHz = 39.3 T lane-ops/s at 2 ops per symbol.
DECODE_VALU_PEAK_SYMS = 256 * 64 * 2.4e9 / 2
# LDS random-gather ceiling (the one that binds): 32 banks of 4 bytes, a wave64 read served as two
# half-waves of 32 lanes; 32 uniformly random requests over 32 banks have an expected largest bank
# load of 3.532, so a half-wave takes 3.532 cycles: 64 / (2 x 3.532) = 9.06 lookups/clk/CU, x 256
# CUs x 2.4 GHz = 5.57 T lookups/s.
LDS_GATHER_PEAK = 256 * 2.4e9 * 64 / (2 * 3.532)
# LUT rung: one conflict-free 4-byte codebook read per two weights (the codebook is replicated
# across the banks); the LDS serves 128 bytes per clock per CU, i.e. 32 such reads: 256 CUs x
# 2.4 GHz x 32 = 19.7 T reads/s (39.3 T weights/s).  It is not what binds that rung: its passes
# wait on the vector-memory path (texture addresser and data return), whose counters are kept
# with the LUT-rung kernel profiles.
LDS_CODEBOOK_PEAK = 256 * 2.4e9 * 32
SWEEP_N = [8, 16, 32, 64, 128, 256, 512, 683, 1024]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["trellis_quantized_moe_expert_amd/csrc/expert.hip",
                  "trellis_quantized_moe_expert_amd/csrc/expert_body.h",
                  "trellis_quantized_moe_expert_amd/csrc/expert_lut.hip",
                  "trellis_quantized_moe_expert_amd/csrc/qtip_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Runner:
    """Plan + device weights + workspace; forwards one batch through the C ABI."""

    def __init__(self, inp, arm, max_tokens, out_dtype, weights=None, variant=0, act_layout=0, small_batch="fused"):
        import torch
        import trellis_quantized_moe_expert_amd as q
        from moe_inputs.device import weights_to_device
        self.q = q
        s = inp.shape
        self.shape = s
        arm_code = {"auto": q.QTIP_ARM_AUTO, "gemv": q.QTIP_ARM_GEMV, "grouped": q.QTIP_ARM_GROUPED,
                    "dequant": q.QTIP_ARM_DEQUANT}[arm]
        od = q.QTIP_OUT_BF16 if out_dtype == "bf16" else q.QTIP_OUT_F32
        rung = q.QTIP_RUNG_LUT if s.rung == "lut" else q.QTIP_RUNG_BITSHIFT
        sb = q.QTIP_SMALL_BATCH_SEPARATE if small_batch == "separate" else q.QTIP_SMALL_BATCH_FUSED
        self.plan = q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, max_tokens, arm_code,
                                                variant, od, 0, act_layout=act_layout, rung=rung,
                                                small_batch=sb), 0)
        self.info = q.qtip_moe_plan_info(self.plan)
        self.ws = torch.empty(self.info["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
        self.dw = weights if weights is not None else weights_to_device(inp)
        d = self.dw
        self.w = q.make_weights(d.codes_gate, d.codes_up, d.codes_down, d.scale_gate, d.scale_up, d.scale_down, d.lut)
        self.out_dtype = torch.int16 if out_dtype == "bf16" else torch.float32
        self.stream = torch.cuda.current_stream()

    def bind(self, inp):
        import torch
        from moe_inputs.device import tokens_to_device
        self.n = inp.logits.shape[0]
        self.tok = tokens_to_device(inp)
        self.out = torch.empty((self.n, self.shape.hidden), dtype=self.out_dtype, device="cuda:0")

    def step(self):
        self.q.qtip_moe_forward(self.plan, self.w, self.tok.x, self.tok.logits, self.n, self.out, self.ws,
                                self.ws.numel(), self.stream)

    def routing_counts(self):
        """Per-expert pair counts of the bound batch, from the GPU router."""
        import torch
        q, s, n = self.q, self.shape, self.n
        dev = lambda *shape, dt=torch.int32: torch.empty(shape, dtype=dt, device="cuda:0")
        idx, w = dev(n, s.top_k), dev(n, s.top_k, dt=torch.float32)
        counts, offs, sp, tm, nt = dev(s.num_experts), dev(s.num_experts + 1), dev(n * s.top_k), dev(n * s.top_k, 3), dev(1)
        q.qtip_moe_route(self.plan, self.tok.logits, n, idx, w, counts, offs, sp, tm, nt, self.stream)
        torch.cuda.synchronize()
        return counts.cpu().numpy(), int(nt.cpu().numpy()[0])

    def close(self):
        self.q.qtip_moe_plan_destroy(self.plan)


def timed(runner, steps, warmup, profile=True):
    import torch
    q = runner.q
    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    if profile:
        q.qtip_moe_profile_enable(runner.plan, min(steps, 4096))
    q.qtip_moe_stats_reset(runner.plan)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()          # single process: the barrier is this synchronisation
    t0 = time.perf_counter()
    ev0.record(runner.stream)
    for _ in range(steps):
        runner.step()
    ev1.record(runner.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stats = q.qtip_moe_stats(runner.plan)
    prof = q.qtip_moe_profile_read(runner.plan) if profile else None
    if profile:
        q.qtip_moe_profile_enable(runner.plan, 0)
    return {"wall_s": t1 - t0, "gpu_ms": ev0.elapsed_time(ev1), "stats": stats, "prof": prof}


def measure_graph(runner, steps, warmup=5):
    """The same forward captured once in a HIP graph and replayed `steps` times (HIP events on
    the replay stream): what a serving loop that captures the layer sees, without per-kernel
    launch costs.  Reported beside the eager figure, not as it."""
    import torch
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            runner.q.qtip_moe_forward(runner.plan, runner.w, runner.tok.x, runner.tok.logits, runner.n, runner.out,
                                      runner.ws, runner.ws.numel(), cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    del g
    return {"ms_per_step": ms, "tokens_per_s": runner.n / (ms * 1e-3), "steps": steps}


def measure_router(runner, inp, calls=200, layers=50):
    """Router GEMM (qtip_moe_router_logits) per-call time from HIP events on the launch stream,
    and the layer from hidden states (qtip_moe_forward_hidden) in tokens/s, on this batch."""
    import numpy as np
    import torch
    import moe_inputs
    q, s, n = runner.q, runner.shape, runner.n
    w = moe_inputs.make_router_weight(s, seed=0)
    w_dev = torch.from_numpy(w.view(np.int16)).to("cuda:0")
    lg = torch.empty((n, s.num_experts), dtype=torch.float32, device="cuda:0")
    call = lambda: q.qtip_moe_router_logits(runner.plan, runner.tok.x, w_dev, n, lg, runner.ws, runner.ws.numel(),
                                            runner.stream)
    layer = lambda: q.qtip_moe_forward_hidden(runner.plan, runner.w, w_dev, runner.tok.x, n, runner.out, runner.ws,
                                              runner.ws.numel(), runner.stream)
    for _ in range(10):
        call()
        layer()
    torch.cuda.synchronize()
    q.qtip_moe_stats_reset(runner.plan)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record(runner.stream)
    for _ in range(calls):
        call()
    e[1].record(runner.stream)
    e[2].record(runner.stream)
    for _ in range(layers):
        layer()
    e[3].record(runner.stream)
    torch.cuda.synchronize()
    st = q.qtip_moe_stats(runner.plan)
    if st["router_launches"] != calls + layers or st["forward_calls"] != layers:
        print(f"bench: router counters do not match the calls made: {st}", file=sys.stderr)
        sys.exit(2)
    call_s = e[0].elapsed_time(e[1]) * 1e-3 / calls
    layer_s = e[2].elapsed_time(e[3]) * 1e-3 / layers
    S = q.qtip_moe_router_split(runner.plan, n)
    flops = 2.0 * n * s.hidden * s.num_experts
    nbytes = 2.0 * s.num_experts * s.hidden + 2.0 * n * s.hidden + 4.0 * n * s.num_experts
    if S > 1:
        nbytes += 2 * 4.0 * S * n * s.num_experts     # partial sums written, then read by the reduction
    return {"split": S, "us_per_call": call_s * 1e6, "flops": flops, "tflops": flops / call_s / 1e12,
            "mfma_bf16_frac": flops / call_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, "bytes": nbytes,
            "gbs": nbytes / call_s / 1e9, "hbm_frac": nbytes / call_s / 1e9 / HBM_PEAK_GBS,
            "forward_hidden_ms": layer_s * 1e3, "forward_hidden_tokens_per_s": n / layer_s}


def schedule_figures(counts, shape, arm, sched):
    """Algorithmic bytes and symbols of one forward, from the router's per-expert counts and the
    plan's schedule (how many binned pairs share one decode of an expert's rows)."""
    import numpy as np
    E, H, I = shape.num_experts, shape.hidden, shape.inter
    woken = int((counts > 0).sum())
    per_expert_bytes = {"gate_up": 2 * I * H // 4 + 2 * I * 2, "down": H * I // 4 + H * 2}

    def decodes_for(per):  # each pass's units hold up to `per` pairs: one decode each
        return int(sum((c + per - 1) // per for c in counts.tolist()))

    dec = {"gate_up": decodes_for(sched["gate_up"]["pairs_per_decode"]),
           "down": decodes_for(sched["down"]["pairs_per_decode"])}
    return {"woken": woken, "units": dict(dec), "decodes": dec,
            "bytes": {k: woken * v for k, v in per_expert_bytes.items()},
            "symbols_min": {"gate_up": woken * 2 * I * H, "down": woken * H * I},
            "symbols_sched": {"gate_up": dec["gate_up"] * 2 * I * H, "down": dec["down"] * H * I},
            "max_count": int(np.max(counts))}


def read_traffic(workload, arm):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{workload}/{arm}/gate_up"
    ent = rec.get(key)
    if not ent or ent.get("kernel_source_sha") != kernel_source_sha():
        return None       # counters were taken on another version of the kernel
    return ent.get("hbm_bytes_per_launch")


def summarize_traffic(fetch_csv, write_csv, workload, arm, command):
    """HBM bytes per launch of the gate+up kernel from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch), each scaled by what the counter reads for the 1 GiB device copy
    that --calibrate-copy runs in the same process.  Writes an entry of profiles/traffic.json."""
    import csv
    copy_bytes = 1 << 30

    def read(path, counter):
        calib, vals = 0.0, []
        mode_digit = "1" if arm == "grouped" else "0"
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name:
                calib = max(calib, v)
            elif re.search(rf"expert_kernel<0, {mode_digit}[,>]", name):
                vals.append(v)
        if calib <= 0 or not vals:
            raise SystemExit(f"{path}: no calibration copy or no gate+up dispatch for {counter}")
        return sum(vals) / len(vals), copy_bytes / (calib * 1024.0), len(vals)

    fetch, f_fetch, nf = read(fetch_csv, "FETCH_SIZE")
    write, f_write, nw = read(write_csv, "WRITE_SIZE")
    ent = {"kernel_source_sha": kernel_source_sha(), "fetch_kib": fetch, "write_kib": write,
           "fetch_factor": f_fetch, "write_factor": f_write, "dispatches": [nf, nw],
           "hbm_bytes_per_launch": fetch * 1024.0 * f_fetch + write * 1024.0 * f_write, "command": command}
    rec = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    rec[f"{workload}/{arm}/gate_up"] = ent
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    log(json.dumps(ent))


def measure_gather_ceiling(rounds=2000):
    import torch
    import trellis_quantized_moe_expert_amd as q
    n = torch.cuda.get_device_properties(0).multi_processor_count * 1024
    sink = torch.empty(n, dtype=torch.int32, device="cuda:0")
    return q.qtip_measure_lut_gather(rounds, sink, n, torch.cuda.current_stream())


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, n_experts=-1):
    """The oracle as it stands (declared mode, numpy float64) over a process pool on the host's
    cores, one BLAS thread per worker: routing and binning of the batch, each woken expert
    decoded once and evaluated on all its pairs, and the combine.  n_experts < 0 times the whole
    layer; otherwise only the first n_experts woken experts are evaluated (no combine) and the
    time is scaled to every woken expert.  Must run before this process touches the GPU (the
    pool forks)."""
    import numpy as np
    from oracle import pool, routing
    s = inp.shape
    idx, _ = routing.route_topk(inp.logits, s.top_k)
    woken = [int(e) for e in np.nonzero(np.bincount(idx.reshape(-1), minlength=s.num_experts))[0]]
    whole = n_experts < 0 or n_experts >= len(woken)
    sample = woken if whole else woken[:max(1, n_experts)]
    workers = pool.default_workers()
    split = {}
    t0 = time.perf_counter()
    pool.layer_outputs({"layer": inp}, workers, experts=None if whole else sample, timing=split)
    dt = time.perf_counter() - t0
    full_s = dt * len(woken) / len(sample)
    what = (f"the whole {s.n_tokens}-token layer (routing and binning, all {len(woken)} woken experts each "
            f"decoded once and evaluated on all its pairs, the combine)" if whole else
            f"{len(sample)} of the {len(woken)} woken experts of this {s.n_tokens}-token batch (routing and "
            f"binning of the whole batch, then each sampled expert decoded once and evaluated on all its "
            f"pairs), scaled by {len(woken)}/{len(sample)} to the whole layer")
    return {"value": s.n_tokens / full_s, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{what}; {dt:.1f} s wall on {workers} worker processes with one BLAS thread each",
            "host": {"os_cpu_count": os.cpu_count(), "workers": workers, "blas_threads_per_worker": 1,
                     "cpu_model": cpu_model()},
            "seconds_measured": dt, "seconds_layer": full_s,
            # worker seconds (summed over the pool) spent decoding the experts' weights and in the
            # matmuls of their pairs; the rest of the wall time is routing, binning, the combine and
            # the pool itself
            "worker_seconds": {"decode": split.get("decode_s"), "matmul": split.get("pairs_s")}}


def calibrate_copy():
    import torch
    nbytes = 1 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"calibrate-copy: copied {nbytes} bytes device to device")
    del a, b


def run_sweep(path, steps, warmup, variant=0, arms=("gemv", "grouped"), n_list=None, layouts=(0,), rung="bitshift",
              small_batch="fused"):
    import moe_inputs
    shape = moe_inputs.WORKLOADS["v4_decode_n32" if rung == "bitshift" else "lut_v4_decode_n32"]
    log("sweep: drawing V4-shaped weights once")
    n_list = n_list or SWEEP_N
    inps = moe_inputs.make_inputs_multi(shape, n_list, seed=0)
    base = None
    with open(path, "a") as f:
        for arm, layout in [(a, l) for a in arms for l in layouts]:
            r = Runner(inps[n_list[0]], arm, max(n_list), "bf16", weights=base, variant=variant, act_layout=layout,
                       small_batch=small_batch)
            base = r.dw
            for n in n_list:
                r.bind(inps[n])
                res = timed(r, steps, warmup, profile=False)
                prof = timed(r, steps, 1, profile=True)["prof"]
                counts, _ = r.routing_counts()
                sched = r.q.qtip_moe_plan_schedule(r.plan, n)
                fig = schedule_figures(counts, r.shape, arm, sched)
                ms = res["wall_s"] * 1e3 / steps
                rec = {"rung": rung, "arm": arm, "n": n, "variant_requested": variant, "act_layout": layout,
                       "small_batch": small_batch,
                       "ms_per_step": ms,
                       "tokens_per_s": n / (ms * 1e-3),
                       "stage_ms": {k: v / prof["n_forwards"] for k, v in prof.items() if k != "n_forwards"},
                       "launches": {k: res["stats"][k] for k in ("gemv_launches", "grouped_launches",
                                                                 "dequant_launches")},
                       "woken": fig["woken"], "decodes": fig["decodes"], "schedule": sched,
                       "predicate_grouped": r.q.qtip_fill_select_grouped(n, 6, 256, 16)}
                f.write(json.dumps(rec) + "\n")
                f.flush()
                log(json.dumps(rec))
            r.close()


HEADLINE = "v4_full_n1024"
CURVE = ["v4_decode_n1", "v4_decode_n32", "v4_mid_n128", "v4_mid_n512", "v4_full_n683", "v4_zipf_n256", "tiny",
         # the LUT rung (a 512 x 2 codebook per layer) on the same layer shapes
         "lut_v4_decode_n1", "lut_v4_decode_n32", "lut_v4_mid_n128", "lut_v4_full_n1024"]


def draw_layers(names):
    """Seeded inputs for each workload; the V4 layers of one rung with uniform routing share one
    weight draw (the draw make_workload makes for each of them), so the device holds one copy of
    each rung's weights."""
    import moe_inputs
    W = moe_inputs.WORKLOADS
    out = {}
    for rung in ("bitshift", "lut"):
        shared = [n for n in names if W[n].num_experts == 256 and W[n].routing == "uniform" and W[n].rung == rung]
        if shared:
            multi = moe_inputs.make_inputs_multi(W[shared[0]], sorted({W[n].n_tokens for n in shared}), seed=0)
            out.update({n: multi[W[n].n_tokens] for n in shared})
    for n in names:
        if n not in out:
            out[n] = moe_inputs.make_workload(n, seed=0)
    return out


def decode_roofline(rung, gu_syms, layer_syms, gather_measured):
    """The decode's own ceiling for decoded weights per second of the gate+up pass and of both
    expert passes: bitshift rung, one random LDS gather per weight (model and measured ceilings);
    LUT rung, one conflict-free codebook read per two weights."""
    if rung == "lut":
        return {"bound": "lds_codebook", "unit": "codebook reads/s (two weights each)",
                "gate_up_achieved": gu_syms / 2, "expert_passes_achieved": layer_syms / 2,
                "peak_model": LDS_CODEBOOK_PEAK, "gate_up_frac_model": gu_syms / 2 / LDS_CODEBOOK_PEAK,
                "expert_passes_frac_model": layer_syms / 2 / LDS_CODEBOOK_PEAK,
                "binding": "vector-memory path (texture addresser and data return), not the LDS"}
    return {"bound": "lds_gather", "unit": "LUT lookups/s",
            "gate_up_achieved": gu_syms, "expert_passes_achieved": layer_syms,
            "peak_measured": gather_measured, "gate_up_frac_measured": gu_syms / gather_measured,
            "expert_passes_frac_measured": layer_syms / gather_measured,
            "peak_model": LDS_GATHER_PEAK, "gate_up_frac_model": gu_syms / LDS_GATHER_PEAK,
            "valu_peak": DECODE_VALU_PEAK_SYMS, "gate_up_frac_valu": gu_syms / DECODE_VALU_PEAK_SYMS,
            "expert_passes_frac_valu": layer_syms / DECODE_VALU_PEAK_SYMS}


def measure_workload(name, inp, weights, args, gather_measured, full=False):
    """Times one workload in the plan a caller of that size uses (max_tokens = n, automatic arm
    unless --arm, bf16 output unless --out-dtype) and returns its record."""
    s = inp.shape
    runner = Runner(inp, args.arm, s.n_tokens, args.out_dtype, weights=weights, variant=args.variant,
                    small_batch=args.small_batch)
    runner.bind(inp)
    q = runner.q
    arm_code = q.qtip_moe_select_arm(runner.plan, s.n_tokens)
    arm = {q.QTIP_ARM_GROUPED: "grouped", q.QTIP_ARM_DEQUANT: "dequant"}.get(arm_code, "gemv")
    q.qtip_moe_log_engaged(runner.plan, s.n_tokens)
    # the timed loop records no stage events (they would add gaps between the kernels); the stage
    # breakdown comes from a second, profiled loop of the same forward
    res = timed(runner, args.steps, args.warmup, profile=False)
    res["prof"] = timed(runner, min(args.steps, 100), 2, profile=True)["prof"]
    counts, n_tiles = runner.routing_counts()
    sched = q.qtip_moe_plan_schedule(runner.plan, s.n_tokens)
    extra = {}
    if full:
        extra["router_gemm"] = measure_router(runner, inp)
        extra["graph_replay"] = measure_graph(runner, args.steps)
    runner.close()
    if res["wall_s"] <= 0 or res["prof"]["n_forwards"] <= 0:
        print(f"bench: no time or no profiled forwards recorded for {name}", file=sys.stderr)
        sys.exit(2)
    counters = res["stats"]
    want = {"grouped": ("grouped_launches", 2), "gemv": ("gemv_launches", 2), "dequant": ("dequant_launches", 4)}[arm]
    vkey = {"grouped": "grouped_variant_launches", "gemv": "gemv_variant_launches"}.get(arm)
    variants_ok = vkey is None or all(counters[vkey][sched[p]["variant"]] >= args.steps for p in ("gate_up", "down"))
    if counters[want[0]] != want[1] * args.steps or not variants_ok:
        print(f"bench: launch counters do not show the {arm} arm and its configurations for {name}: {counters}",
              file=sys.stderr)
        sys.exit(2)
    fig = schedule_figures(counts, s, arm, sched)
    nf = res["prof"]["n_forwards"]
    stage_ms = {k: v / nf for k, v in res["prof"].items() if k != "n_forwards"}
    ms_per_step = res["wall_s"] * 1e3 / args.steps
    layer_gpu_s = res["gpu_ms"] * 1e-3 / args.steps
    gu_s, dn_s = stage_ms["gate_up"] * 1e-3, stage_ms["down"] * 1e-3
    gu_gbs = fig["bytes"]["gate_up"] / gu_s / 1e9
    layer_bytes = fig["bytes"]["gate_up"] + fig["bytes"]["down"]
    gu_syms = fig["symbols_sched"]["gate_up"] / gu_s
    layer_syms = (fig["symbols_sched"]["gate_up"] + fig["symbols_sched"]["down"]) / (gu_s + dn_s)
    flops = 6.0 * s.n_tokens * s.top_k * s.hidden * s.inter
    rec = {
        "workload": name, "n_tokens": s.n_tokens, "routing": s.routing, "rung": s.rung,
        "shape": {"experts": s.num_experts, "top_k": s.top_k, "hidden": s.hidden, "inter": s.inter},
        "arm": arm, "variant": {"gate_up": sched["gate_up"]["variant"], "down": sched["down"]["variant"]},
        "tokens_per_s": s.n_tokens * args.steps / res["wall_s"], "ms_per_step": ms_per_step,
        "gpu_event_ms_per_step": layer_gpu_s * 1e3, "stage_ms": stage_ms,
        "gate_up_packed_bytes": fig["bytes"]["gate_up"], "down_packed_bytes": fig["bytes"]["down"],
        "gate_up_packed_gbs": gu_gbs, "gate_up_hbm_frac": gu_gbs / HBM_PEAK_GBS,
        "layer_packed_gbs": layer_bytes / layer_gpu_s / 1e9,
        "layer_hbm_frac": layer_bytes / layer_gpu_s / 1e9 / HBM_PEAK_GBS,
        "woken_experts": fig["woken"], "max_pairs_per_expert": fig["max_count"], "m_tiles": n_tiles,
        "decodes": fig["decodes"],
        "decode_roofline": decode_roofline(s.rung, gu_syms, layer_syms, gather_measured),
        # MFMA work of the layer (g, u and y: 2 n k H I flops each) against the dense bf16 peak: the
        # contraction is thin, so this stays a few percent at most
        "mfma": {"flops": flops, "layer_tflops": flops / layer_gpu_s / 1e12,
                 "layer_frac": flops / layer_gpu_s / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "schedule": sched,
        "launch_counters": {k: counters[k] for k in ("gemv_launches", "grouped_launches", "dequant_launches",
                                                     "route_launches", "combine_launches", "router_launches",
                                                     "routed_in_gate_up", "combined_in_down",
                                                     "gemv_variant_launches", "grouped_variant_launches")},
    }
    rec.update(extra)
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--curve", default=",".join(CURVE), help="comma-separated workloads measured beside the "
                    "headline and reported in detail.curve ('' for none)")
    ap.add_argument("--arm", choices=["auto", "gemv", "grouped", "dequant"], default="auto")
    ap.add_argument("--small-batch", choices=["fused", "separate"], default="fused",
                    help="small GEMV batches in two launches (routing in the gate+up launch, combine in the down "
                    "launch) or in four")
    ap.add_argument("--out-dtype", choices=["bf16", "f32"], default="bf16")
    ap.add_argument("--variant", type=int, default=0, help="expert kernel variant (0 = the plan's choice, 1..11 fixed; see qtip_moe_plan_schedule)")
    ap.add_argument("--cpu-experts", type=int, default=-1, help="woken experts the CPU oracle is timed on (-1: the "
                    "whole layer, about 13 s on 16 cores at n=1024; 0: skip)")
    ap.add_argument("--sweep", metavar="PATH", default=None)
    ap.add_argument("--sweep-arms", default="gemv,grouped")
    ap.add_argument("--sweep-layouts", default="0", help="grouped-arm activation layouts to sweep (0 auto, 1 rows, "
                    "2 fragments)")
    ap.add_argument("--sweep-n", default=None, help="comma-separated token counts (default: the fixed list)")
    ap.add_argument("--sweep-rung", choices=["bitshift", "lut"], default="bitshift")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter_collection files")
    ap.add_argument("--traffic-command", default="", help="the profiling command, recorded with --traffic-from")
    args = ap.parse_args()

    if args.traffic_from:
        summarize_traffic(args.traffic_from[0], args.traffic_from[1], args.workload,
                          "grouped" if args.arm == "grouped" else args.arm, args.traffic_command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the path is measured on one GPU's share and has no multi-GPU "
              f"mode; got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        sys.exit(2)
    import moe_inputs
    if args.sweep:
        import torch
        if not torch.cuda.is_available():
            print("no GPU visible", file=sys.stderr)
            sys.exit(2)
        if args.calibrate_copy:
            calibrate_copy()
        n_list = [int(x) for x in args.sweep_n.split(",")] if args.sweep_n else None
        run_sweep(args.sweep, args.steps, args.warmup, args.variant, tuple(args.sweep_arms.split(",")), n_list,
                  tuple(int(x) for x in args.sweep_layouts.split(",")), args.sweep_rung, args.small_batch)
        return

    curve = [c for c in args.curve.split(",") if c and c != args.workload]
    for name in [args.workload] + curve:
        if name not in moe_inputs.WORKLOADS:
            print(f"unknown workload {name!r}", file=sys.stderr)
            sys.exit(2)
    log(f"bench: drawing workloads {[args.workload] + curve}")
    layers = draw_layers([args.workload] + curve)
    # the CPU oracle runs first: its worker pool forks, and this process has not touched the GPU yet
    cpu = cpu_baseline(layers[args.workload], args.cpu_experts) if args.cpu_experts != 0 else None
    if cpu:
        log(f"bench: cpu baseline {cpu['value']:.3f} tokens/s ({cpu['sample']})")

    import torch
    from moe_inputs.device import weights_to_device
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
    gather_measured = measure_gather_ceiling()
    import numpy as np
    dev_weights = []   # (host inputs, device weights): one device copy per distinct weight draw
    fields = ("lut", "codes_gate", "codes_up", "codes_down", "scale_gate", "scale_up", "scale_down")

    def weights_for(name):
        inp = layers[name]
        for host, dw in dev_weights:
            if all(getattr(host, f).shape == getattr(inp, f).shape and np.array_equal(getattr(host, f), getattr(inp, f))
                   for f in fields):
                return dw
        dw = weights_to_device(inp)
        dev_weights.append((inp, dw))
        return dw

    head = measure_workload(args.workload, layers[args.workload], weights_for(args.workload), args, gather_measured,
                            full=True)
    points = []
    for name in curve:
        log(f"bench: curve point {name}")
        points.append(measure_workload(name, layers[name], weights_for(name), args, gather_measured))
    s = layers[args.workload].shape
    line = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "experts": s.num_experts, "top_k": s.top_k, "hidden": s.hidden,
                   "inter": s.inter, "n_tokens": s.n_tokens, "routing": s.routing, "seed": 0, "arm": head["arm"],
                   "out_dtype": args.out_dtype, "max_tokens": s.n_tokens, "variant": head["variant"]},
        "roofline": {"bound": "hbm", "achieved": head["gate_up_packed_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["gate_up_packed_gbs"] / HBM_PEAK_GBS,
                     "traffic": read_traffic(args.workload, head["arm"])},
        "cpu_baseline": cpu,
        "detail": {"dominant_kernel": f"expert_kernel gate+up ({head['arm']} arm)", "headline": head,
                   "curve": points, "gather_ceiling_measured": gather_measured,
                   "kernel_source_sha": kernel_source_sha()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
