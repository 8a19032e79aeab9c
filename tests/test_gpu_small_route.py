"""Small GEMV-arm batches routed and binned inside the fused gate+up launch (route_launch AUTO)
against the same batches routed by the separate routing kernels (route_launch SEPARATE).

The routing and the binning are exact integer work, so the two plans must give the same outputs
bit for bit, in f32 and in bf16; the fused plan must also meet the oracle's bar (fp32 max-abs 2e-2,
rel-L2 1e-3), and the launch counters must show which path ran.  Cases: one to sixteen tokens
(64 pairs at most), every token routed to the same experts (bins of many pairs, cut into several
units per expert in each pass), a router wider than 256 experts (16 logits per lane), logits
given as the router GEMM's partial sums (a forward from hidden states), and both rungs."""
import dataclasses

import numpy as np
import pytest

import moe_inputs
import parity
import trellis_quantized_moe_expert_amd as q
from gpu_util import rung_code, say
from moe_inputs.device import tokens_to_device, weights_to_device
from oracle import moe

pytestmark = pytest.mark.gpu

MID = moe_inputs.MoEShape(num_experts=16, top_k=4, hidden=512, inter=256, n_tokens=16)
MID_LUT = dataclasses.replace(MID, rung="lut")
WIDE = moe_inputs.MoEShape(num_experts=600, top_k=8, hidden=256, inter=128, n_tokens=8)
V4 = moe_inputs.WORKLOADS["v4_decode_n32"]


def plan_for(s, n_max, out_dtype, route_launch):
    od = q.QTIP_OUT_F32 if out_dtype == "f32" else q.QTIP_OUT_BF16
    return q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, n_max, q.QTIP_ARM_GEMV, 0, od,
                                       rung=rung_code(s), route_launch=route_launch), 0)


def run(plan, w, inp, out_dtype, w_router=None):
    """One forward; returns the output (f32 values or bf16 bits) and the plan's counters."""
    import torch
    ws = torch.empty(q.qtip_moe_plan_info(plan)["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
    t = tokens_to_device(inp)
    n = inp.logits.shape[0]
    dt = torch.float32 if out_dtype == "f32" else torch.int16
    out = torch.full((n, inp.shape.hidden), -1, dtype=dt, device="cuda:0")
    q.qtip_moe_stats_reset(plan)
    if w_router is None:
        q.qtip_moe_forward(plan, w, t.x, t.logits, n, out, ws, ws.numel())
    else:
        q.qtip_moe_forward_hidden(plan, w, w_router, t.x, n, out, ws, ws.numel())
    torch.cuda.synchronize()
    a = out.cpu().numpy()
    return (a if out_dtype == "f32" else a.view(np.uint16)), q.qtip_moe_stats(plan)


def both_paths(inp, out_dtype, w_router=None):
    s = inp.shape
    n = inp.logits.shape[0]
    dw = weights_to_device(inp)
    w = q.make_weights(dw.codes_gate, dw.codes_up, dw.codes_down, dw.scale_gate, dw.scale_up, dw.scale_down, dw.lut)
    res = {}
    for route_launch in (q.QTIP_ROUTE_AUTO, q.QTIP_ROUTE_SEPARATE):
        plan = plan_for(s, n, out_dtype, route_launch)
        try:
            fused = q.qtip_moe_plan_schedule(plan, n)["route_in_gate_up"]
            assert fused == (1 if route_launch == q.QTIP_ROUTE_AUTO else 0)
            res[route_launch] = run(plan, w, inp, out_dtype, w_router)
        finally:
            q.qtip_moe_plan_destroy(plan)
    (got, st), (sep, st_sep) = res[q.QTIP_ROUTE_AUTO], res[q.QTIP_ROUTE_SEPARATE]
    assert st["routed_in_gate_up"] == 1 and st["route_launches"] == 0 and st["gemv_launches"] == 2
    assert st_sep["routed_in_gate_up"] == 0 and st_sep["route_launches"] >= 1
    assert st["last_arm"] == st_sep["last_arm"] == q.QTIP_ARM_GEMV
    assert np.array_equal(got.view(np.uint32) if out_dtype == "f32" else got,
                          sep.view(np.uint32) if out_dtype == "f32" else sep)
    return got


CASES = [("mid", MID, 1), ("mid", MID, 3), ("mid", MID, 7), ("mid", MID, 16),
         ("wide", WIDE, 1), ("wide", WIDE, 5), ("wide", WIDE, 8),
         ("mid_lut", MID_LUT, 1), ("mid_lut", MID_LUT, 6), ("mid_lut", MID_LUT, 16)]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,shape,n", CASES)
def test_fused_routing_matches_the_routing_kernels_and_the_oracle(name, shape, n, out_dtype):
    inp = moe_inputs.make_inputs(shape, seed=21, n_tokens=n)
    say(f"small-batch routing {name} n={n} out={out_dtype}")
    got = both_paths(inp, out_dtype)
    ref = moe.moe_forward(inp, out_dtype=out_dtype)
    ok, st = parity.check_f32(got, ref["out_f64"]) if out_dtype == "f32" else parity.check_bf16(got, ref["out"])
    assert ok, st


@pytest.mark.parametrize("name,shape,n", [("mid", MID, 16), ("mid_lut", MID_LUT, 16), ("wide", WIDE, 8)])
def test_every_token_on_the_same_experts(name, shape, n):
    """Identical logit rows: each selected expert holds all n pairs, cut into several units."""
    inp = moe_inputs.make_inputs(shape, seed=22, n_tokens=n)
    inp = dataclasses.replace(inp, logits=np.repeat(inp.logits[:1], n, axis=0))
    say(f"small-batch routing, one expert set {name} n={n}")
    got = both_paths(inp, "f32")
    ref = moe.moe_forward(inp)
    assert ref["bins"]["counts"].max() == n
    ok, st = parity.check_f32(got, ref["out_f64"])
    assert ok, st


@pytest.mark.parametrize("n", [1, 7, 10])
def test_v4_layer_both_routing_paths_agree(n):
    """The V4 layer (256 experts, top-6) at the batch sizes the GEMV arm serves, and n=10 (60
    pairs) on the pinned GEMV arm; the oracle's full comparison at these sizes is elsewhere."""
    inp = moe_inputs.make_inputs(V4, seed=23, n_tokens=n)
    say(f"small-batch routing V4 n={n}")
    both_paths(inp, "bf16")


@pytest.mark.parametrize("name,shape,n", [("v4", V4, 1), ("v4", V4, 4), ("mid", MID, 9)])
def test_forward_from_hidden_states_routes_the_same_either_way(name, shape, n):
    """Logits as the router GEMM's partial sums (added in ascending chunk order by the routing)."""
    import torch
    inp = moe_inputs.make_inputs(shape, seed=24, n_tokens=n)
    w_router = moe_inputs.make_router_weight(shape, seed=24)
    w_dev = torch.from_numpy(np.ascontiguousarray(w_router).view(np.int16)).to("cuda:0")
    say(f"small-batch routing from hidden states {name} n={n}")
    both_paths(inp, "f32", w_router=w_dev)
