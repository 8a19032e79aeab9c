"""Small GEMV-arm batches with the launches folded together (small_batch FUSED: routed and binned
inside the gate+up launch, and, where the down pass's token tasks fit one round on the GPU,
combined inside the down launch) against the same batches with the separate routing and combine
kernels (small_batch SEPARATE).

Routing and binning are exact integer work, and the fused combine adds the same terms in the same
order as the combine kernel (ascending s within a pair, then ascending j); only the down pass's
input split may differ (the token tasks split every row's inputs over S waves, the separate down
pass only when its launch is small), and with it the order of the fp32 additions inside a dot
product.  So the two plans must agree bit for bit where both split alike (every case below but the
V4 layer's single token, whose token tasks halve each row's inputs), and within a few fp32
roundings there; the fused plan must also meet the oracle's bar (fp32 max-abs 2e-2, rel-L2 1e-3;
bf16 within 2e-2 or one bf16 ulp per element, rel-L2 1e-3), and the launch counters and the
schedule must agree on which path ran.  Cases: one to sixteen tokens (64 pairs at most), every
token routed to the same experts (bins of many pairs, cut into several units per expert), a router
wider than 256 experts (16 logits per lane), logits given as the router GEMM's partial sums (a
forward from hidden states), and both rungs."""
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
V4_LUT = moe_inputs.WORKLOADS["lut_v4_decode_n32"]


def plan_for(s, n_max, out_dtype, small_batch):
    od = q.QTIP_OUT_F32 if out_dtype == "f32" else q.QTIP_OUT_BF16
    return q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, n_max, q.QTIP_ARM_GEMV, 0, od,
                                       rung=rung_code(s), small_batch=small_batch), 0)


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


def bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def one_round(s, n):
    """The token tasks (one per token and 16-row block) fit one round on the 256 CUs."""
    return n * (s.hidden // 16) <= 256


def both_paths(inp, out_dtype, w_router=None, exact=True):
    s = inp.shape
    n = inp.logits.shape[0]
    combine = 1 if one_round(s, n) else 0
    dw = weights_to_device(inp)
    w = q.make_weights(dw.codes_gate, dw.codes_up, dw.codes_down, dw.scale_gate, dw.scale_up, dw.scale_down, dw.lut)
    res = {}
    for sb in (q.QTIP_SMALL_BATCH_FUSED, q.QTIP_SMALL_BATCH_SEPARATE):
        plan = plan_for(s, n, out_dtype, sb)
        try:
            sched = q.qtip_moe_plan_schedule(plan, n)
            want = (1, combine) if sb == q.QTIP_SMALL_BATCH_FUSED else (0, 0)
            assert (sched["route_in_gate_up"], sched["combine_in_down"]) == want
            res[sb] = run(plan, w, inp, out_dtype, w_router)
        finally:
            q.qtip_moe_plan_destroy(plan)
    (got, st), (sep, st_sep) = res[q.QTIP_SMALL_BATCH_FUSED], res[q.QTIP_SMALL_BATCH_SEPARATE]
    assert st["routed_in_gate_up"] == 1 and st["combined_in_down"] == combine
    assert st["route_launches"] == 0 and st["combine_launches"] == 1 - combine and st["gemv_launches"] == 2
    assert st_sep["routed_in_gate_up"] == 0 and st_sep["combined_in_down"] == 0
    assert st_sep["route_launches"] >= 1 and st_sep["combine_launches"] == 1
    assert st["last_arm"] == st_sep["last_arm"] == q.QTIP_ARM_GEMV
    if exact:
        assert np.array_equal(got.view(np.uint32) if out_dtype == "f32" else got,
                              sep.view(np.uint32) if out_dtype == "f32" else sep)
    else:
        a = got if out_dtype == "f32" else bf16_to_f32(got)
        b = sep if out_dtype == "f32" else bf16_to_f32(sep)
        # a few fp32 roundings of the largest output (the additions' order), plus, for bf16, the one
        # ulp that a value lying that close to a rounding midpoint may move by
        tol = 1e-5 * float(np.max(np.abs(b)))
        if out_dtype == "bf16":
            tol = tol + 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b))
        assert np.all(np.abs(a - b) <= tol), float(np.max(np.abs(a - b) - tol))
    return got


CASES = [("mid", MID, 1), ("mid", MID, 3), ("mid", MID, 7), ("mid", MID, 16),
         ("wide", WIDE, 1), ("wide", WIDE, 5), ("wide", WIDE, 8),
         ("mid_lut", MID_LUT, 1), ("mid_lut", MID_LUT, 6), ("mid_lut", MID_LUT, 16)]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,shape,n", CASES)
def test_two_launches_match_four_and_the_oracle(name, shape, n, out_dtype):
    inp = moe_inputs.make_inputs(shape, seed=21, n_tokens=n)
    say(f"small batch {name} n={n} out={out_dtype}")
    got = both_paths(inp, out_dtype)
    ref = moe.moe_forward(inp, out_dtype=out_dtype)
    ok, st = parity.check_f32(got, ref["out_f64"]) if out_dtype == "f32" else parity.check_bf16(got, ref["out"])
    assert ok, st


@pytest.mark.parametrize("name,shape,n", [("mid", MID, 16), ("mid_lut", MID_LUT, 16), ("wide", WIDE, 8)])
def test_every_token_on_the_same_experts(name, shape, n):
    """Identical logit rows: each selected expert holds all n pairs, cut into several units."""
    inp = moe_inputs.make_inputs(shape, seed=22, n_tokens=n)
    inp = dataclasses.replace(inp, logits=np.repeat(inp.logits[:1], n, axis=0))
    say(f"small batch, one expert set {name} n={n}")
    got = both_paths(inp, "f32")
    ref = moe.moe_forward(inp)
    assert ref["bins"]["counts"].max() == n
    ok, st = parity.check_f32(got, ref["out_f64"])
    assert ok, st


@pytest.mark.parametrize("name,shape,n", [("v4", V4, 1), ("v4", V4, 4), ("v4", V4, 7), ("v4", V4, 10),
                                          ("v4_lut", V4_LUT, 1), ("v4_lut", V4_LUT, 3), ("v4_lut", V4_LUT, 5)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_v4_layer_two_launches_match_four(name, shape, n, out_dtype):
    """The V4 layer (256 experts, top-6) at the batch sizes the GEMV arm serves by default, and n=10
    (60 pairs); the oracle's full comparison at these sizes is elsewhere."""
    inp = moe_inputs.make_inputs(shape, seed=23, n_tokens=n)
    say(f"small batch V4 {name} n={n} out={out_dtype}")
    both_paths(inp, out_dtype, exact=(n > 1))


@pytest.mark.parametrize("name,shape,n", [("v4", V4, 1), ("v4", V4, 4), ("mid", MID, 9)])
def test_forward_from_hidden_states_two_launches_match_four(name, shape, n):
    """Logits as the router GEMM's partial sums (added in ascending chunk order by the routing)."""
    import torch
    inp = moe_inputs.make_inputs(shape, seed=24, n_tokens=n)
    w_router = moe_inputs.make_router_weight(shape, seed=24)
    w_dev = torch.from_numpy(np.ascontiguousarray(w_router).view(np.int16)).to("cuda:0")
    say(f"small batch from hidden states {name} n={n}")
    both_paths(inp, "f32", w_router=w_dev, exact=(name != "v4" or n > 1))
