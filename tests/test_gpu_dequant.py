"""The dequantize arm on the GPU (qtip_moe_dequantize, qtip_moe_forward with QTIP_ARM_DEQUANT).

Bars: the materialised weights are bf16(LUT[state]) bit for bit against the oracle's decode
(integer-exact work: one table value per weight); the layer meets the usual parity bar (fp32
outputs max-abs 2e-2 and rel-L2 1e-3; bf16 outputs rel-L2 1e-3 and one bf16 ulp), alone and
when the automatic dispatch picks the arm inside a dequantize window, and the launch counters
show the arm that ran.  Shapes span several tiles with ragged tails, a full V4 expert, and the
V4 decode layer with sampled tokens.
"""
import dataclasses

import numpy as np
import pytest

import moe_inputs
import parity
import trellis_quantized_moe_expert_amd as q
from gpu_util import Layer, say
from oracle import fill, moe, trellis
from oracle.numerics import f64_to_bf16_bits

pytestmark = pytest.mark.gpu

MID = moe_inputs.MoEShape(num_experts=16, top_k=4, hidden=512, inter=256, n_tokens=100)


def dequantized(layer, matrix, expert):
    import torch
    s = layer.shape
    rows, cols = (s.hidden, s.inter) if matrix == 2 else (s.inter, s.hidden)
    out = torch.empty((rows, cols), dtype=torch.int16, device="cuda:0")
    q.qtip_moe_dequantize(layer.plan, layer.w, matrix, expert, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,shape,experts", [("tiny", moe_inputs.WORKLOADS["tiny"], [0, 3, 7]),
                                                ("mid", MID, [0, 15]),
                                                ("v4", moe_inputs.WORKLOADS["v4_decode_n32"], [0, 255])])
def test_dequantize_is_bit_exact(name, shape, experts):
    inp = moe_inputs.make_inputs(shape, seed=2, n_tokens=4)
    layer = Layer(inp, max_tokens=4)
    for e in experts:
        for m, codes in enumerate((inp.codes_gate, inp.codes_up, inp.codes_down)):
            say(f"dequantize {name} expert={e} matrix={m}")
            got = dequantized(layer, m, e)
            want = f64_to_bf16_bits(trellis.decode_declared(trellis.stored_rows(codes[e]), inp.lut))
            ok, st = parity.check_exact(got, want)
            assert ok, st
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    assert st["dequant_launches"] == 3 * len(experts)


def dequant_layer(inp, out_dtype="f32", max_tokens=None):
    return Layer(inp, arm=q.QTIP_ARM_DEQUANT, out_dtype=out_dtype, max_tokens=max_tokens)


def check(gpu, ref, out_dtype):
    if out_dtype == "f32":
        ok, st = parity.check_f32(gpu, ref["out_f64"])
    else:
        ok, st = parity.check_bf16(gpu, ref["out"])
    assert ok, st
    return st


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_tiny_layer_on_the_dequantize_arm(seed, out_dtype):
    inp = moe_inputs.make_workload("tiny", seed=seed)
    say(f"dequantize arm tiny seed={seed} out={out_dtype}")
    layer = dequant_layer(inp, out_dtype)
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    assert st["last_arm"] == q.QTIP_ARM_DEQUANT
    assert st["dequant_launches"] == 4 and st["grouped_launches"] == 0 and st["gemv_launches"] == 0
    check(got, moe.moe_forward(inp, out_dtype=out_dtype), out_dtype)


@pytest.mark.parametrize("n", [1, 9, 100, 300])
def test_mid_layer_on_the_dequantize_arm_ragged(n):
    inp = moe_inputs.make_inputs(MID, seed=3, n_tokens=n)
    say(f"dequantize arm mid n={n}")
    layer = dequant_layer(inp, max_tokens=300)
    got = layer.forward(inp)
    layer.close()
    st = check(got, moe.moe_forward(inp), "f32")
    say(f"  {st}")


WIDE = moe_inputs.MoEShape(num_experts=150, top_k=4, hidden=256, inter=128, n_tokens=40)


@pytest.mark.parametrize("rung", ["bitshift", "lut"])
@pytest.mark.parametrize("n", [3, 40])
def test_dequantize_arm_over_a_wide_router(n, rung):
    """150 experts: the woken ones spread over three 64-expert chunks, the last one partly past E.
    The materialise tasks cover the woken experts only (slot s is the s-th woken expert), so a wrong
    slot-to-expert walk would put another expert's weights under a pair."""
    inp = moe_inputs.make_inputs(dataclasses.replace(WIDE, rung=rung), seed=5, n_tokens=n)
    ref = moe.moe_forward(inp)
    woken = np.flatnonzero(ref["bins"]["counts"] > 0)
    say(f"dequantize arm E=150 {rung} n={n}: {woken.size} woken, first {woken[0]}, last {woken[-1]}")
    layer = dequant_layer(inp, max_tokens=n)
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    # two materialise launches and the two dense expert passes
    assert st["last_arm"] == q.QTIP_ARM_DEQUANT and st["dequant_launches"] == 4
    check(got, ref, "f32")


def test_automatic_dispatch_inside_a_dequantize_window():
    # grouped threshold 8 with traffic ratio 4 on the mid shape (top-4 of 16) opens a window
    shape = MID
    lo = fill.min_tokens_grouped(4, 16, 4)
    hi = fill.min_tokens_grouped(4, 16, 8)
    assert fill.dequant_tokens(4, 16, 8, 4, 400) == list(range(lo, hi))
    n = lo
    inp = moe_inputs.make_inputs(shape, seed=4, n_tokens=n)
    s = inp.shape
    layer = Layer(inp, max_tokens=hi)
    q.qtip_moe_plan_destroy(layer.plan)
    layer.plan = q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, hi, dispatch_tile_m=8,
                                             dequant_traffic_ratio=4), 0)
    import torch
    layer.ws = torch.empty(q.qtip_moe_plan_info(layer.plan)["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
    assert q.qtip_moe_dequant_range(layer.plan) == (lo, hi)
    say(f"automatic dispatch n={n} in window [{lo}, {hi})")
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    assert st["last_arm"] == q.QTIP_ARM_DEQUANT and st["dequant_launches"] == 4
    check(got, moe.moe_forward(inp), "f32")


def test_v4_decode_layer_on_the_dequantize_arm_sampled():
    inp = moe_inputs.make_workload("v4_decode_n32", seed=0)
    say("dequantize arm V4 n=32")
    layer = dequant_layer(inp, max_tokens=32)
    got = layer.forward(inp)
    layer.close()
    toks = [0, 31]
    ref = moe.moe_forward(inp, tokens=toks)
    st = check(got[toks], ref, "f32")
    say(f"  {st}")
