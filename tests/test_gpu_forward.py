"""End-to-end MoE layer on the GPU (qtip_moe_forward) vs the declared-mode oracle.

Bars: fp32 outputs within max-abs 2e-2 and rel-L2 1e-3; bf16 outputs within rel-L2 1e-3 and,
per element, within 2e-2 or one bf16 ulp of the oracle's bf16 value.  Full comparison at sizes the oracle finishes in seconds (several
tiles and ragged tails); at the full workload sizes, in the launch configuration the
benchmark uses, sampled tokens are compared one by one.  Both arms must agree with the
oracle and with each other, and the launch counters must show the arm that ran."""
import dataclasses

import numpy as np
import pytest

import moe_inputs
import parity
import trellis_quantized_moe_expert_amd as q
from gpu_util import Layer, say
from oracle import moe

pytestmark = pytest.mark.gpu

ARMS = [q.QTIP_ARM_AUTO, q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED]


def check(gpu, ref, out_dtype):
    if out_dtype == "f32":
        ok, st = parity.check_f32(gpu, ref["out_f64"])
    else:
        ok, st = parity.check_bf16(gpu, ref["out"])
    assert ok, st
    return st


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("arm", ARMS)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_tiny_workload_full_parity(seed, arm, out_dtype):
    inp = moe_inputs.make_workload("tiny", seed=seed)
    say(f"forward tiny seed={seed} arm={arm} out={out_dtype}")
    layer = Layer(inp, arm=arm, out_dtype=out_dtype)
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    expect_arm = q.qtip_moe_select_arm(layer.plan, 16)
    assert st["last_arm"] == expect_arm
    if expect_arm == q.QTIP_ARM_GROUPED:
        assert st["grouped_launches"] == 2 and st["gemv_launches"] == 0
    else:
        assert st["gemv_launches"] == 2 and st["grouped_launches"] == 0
    layer.close()
    check(got, moe.moe_forward(inp, out_dtype=out_dtype), out_dtype)


MID = moe_inputs.MoEShape(num_experts=16, top_k=4, hidden=512, inter=256, n_tokens=100)


@pytest.mark.parametrize("arm", [q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED])
@pytest.mark.parametrize("n", [1, 9, 100, 300])
def test_mid_shape_full_parity_ragged_tiles(arm, n):
    inp = moe_inputs.make_inputs(MID, seed=3, n_tokens=n)
    say(f"forward mid n={n} arm={arm}")
    layer = Layer(inp, arm=arm, out_dtype="f32", max_tokens=300)
    got = layer.forward(inp)
    layer.close()
    check(got, moe.moe_forward(inp), "f32")


def test_zipf_small_hot_expert_spans_many_units():
    shape = moe_inputs.MoEShape(num_experts=32, top_k=4, hidden=256, inter=128, n_tokens=400, routing="zipf")
    inp = moe_inputs.make_inputs(shape, seed=4)
    say("forward small zipf")
    ref = moe.moe_forward(inp)
    assert ref["bins"]["counts"].max() > 64          # one expert needs several decode units
    for arm in (q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED):
        layer = Layer(inp, arm=arm)
        got = layer.forward(inp)
        layer.close()
        check(got, ref, "f32")


def test_arms_agree_with_each_other():
    inp = moe_inputs.make_inputs(MID, seed=5, n_tokens=200)
    say("forward arms agree")
    outs = []
    for arm in (q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED):
        layer = Layer(inp, arm=arm)
        outs.append(layer.forward(inp))
        layer.close()
    # The arms sum in different orders before h is rounded to bf16, so rare one-ulp flips of
    # h are expected; they are held to the same bar as each arm against the oracle.
    ok, st = parity.check_f32(outs[0], outs[1].astype(np.float64))
    say(f"  GEMV vs grouped: {st}")
    assert ok, st


def test_repeated_calls_and_smaller_second_batch_reuse_workspace():
    inp = moe_inputs.make_inputs(MID, seed=6, n_tokens=120)
    say("forward repeated")
    layer = Layer(inp, arm=q.QTIP_ARM_GROUPED, max_tokens=120)
    a = layer.forward(inp)
    small = moe_inputs.redraw_tokens(inp, 17, seed=7)
    b = layer.forward(small)
    c = layer.forward(inp)
    layer.close()
    assert np.array_equal(a, c)                    # deterministic: same bits every call
    check(b, moe.moe_forward(small), "f32")


V4_SAMPLES = {"v4_decode_n32": [0, 31], "v4_mid_n128": [77], "v4_mid_n512": [500], "v4_full_n683": [682],
              "v4_full_n1024": [1], "v4_zipf_n256": [3, 200]}


@pytest.mark.parametrize("name", list(V4_SAMPLES))
def test_full_size_workloads_sampled_tokens(name):
    inp = moe_inputs.make_workload(name, seed=0)
    n = inp.shape.n_tokens
    say(f"forward full-size {name} n={n}")
    layer = Layer(inp, out_dtype="f32", max_tokens=1024)
    got = layer.forward(inp)
    arm = q.qtip_moe_stats(layer.plan)["last_arm"]
    layer.close()
    assert np.all(np.isfinite(got))
    toks = V4_SAMPLES[name]
    ref = moe.moe_forward(inp, tokens=toks)
    ok, st = parity.check_f32(got[toks], ref["out_f64"])
    say(f"  arm={arm} {st}")
    assert ok, st


def test_v4_small_batches_full_parity():
    """Decode-width batches of the V4 layer on the GEMV arm, whose launches have fewer tasks than
    the GPU has wave slots and run with fewer waves per workgroup on every CU; every token is
    compared."""
    inps = moe_inputs.make_inputs_multi(moe_inputs.WORKLOADS["v4_decode_n32"], [1, 2, 5, 8], seed=21)
    layer = Layer(inps[1], arm=q.QTIP_ARM_GEMV, out_dtype="f32", max_tokens=8)
    for n in (1, 2, 5, 8):
        say(f"forward V4 small batch n={n}")
        got = layer.forward(inps[n])
        assert q.qtip_moe_stats(layer.plan)["last_arm"] == q.QTIP_ARM_GEMV
        check(got, moe.moe_forward(inps[n]), "f32")
    layer.close()


def test_v4_decode_floor_switches_arms_at_eight_tokens():
    """The plan's decode floor (7 by default on the bitshift rung): 7 tokens take the GEMV arm, 8
    the grouped arm; both match the oracle token by token."""
    inps = moe_inputs.make_inputs_multi(moe_inputs.WORKLOADS["v4_decode_n32"], [7, 8], seed=22)
    layer = Layer(inps[7], out_dtype="f32", max_tokens=8)
    for n, arm in ((7, q.QTIP_ARM_GEMV), (8, q.QTIP_ARM_GROUPED)):
        say(f"forward V4 floor n={n}")
        got = layer.forward(inps[n])
        assert q.qtip_moe_stats(layer.plan)["last_arm"] == arm
        check(got, moe.moe_forward(inps[n]), "f32")
    layer.close()


def test_forward_rejects_empty_and_oversized_batches_on_device():
    import torch
    inp = moe_inputs.make_workload("tiny", seed=0)
    layer = Layer(inp)
    out = torch.empty((16, 256), dtype=torch.float32, device="cuda:0")
    for n in (0, 17):
        with pytest.raises(q.QtipError) as ei:
            q.qtip_moe_forward(layer.plan, layer.w, 256, 256, n, out, layer.ws, layer.ws.numel())
        assert ei.value.status == q.QTIP_ERR_INVALID_CONFIG
    layer.close()


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11])
@pytest.mark.parametrize("arm", [q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED])
def test_kernel_variants_full_parity(variant, arm):
    """Both kernel configurations (16 waves / 32-pair decodes, 8 waves / 64-pair decodes) on a
    batch whose experts need several decodes per unit on either arm."""
    inp = moe_inputs.make_inputs(MID, seed=8, n_tokens=260)
    say(f"forward variant={variant} arm={arm}")
    s = inp.shape
    layer = Layer(inp, arm=arm)
    q.qtip_moe_plan_destroy(layer.plan)
    layer.plan = q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, 260, arm, variant,
                                             q.QTIP_OUT_F32, 0), 0)
    got = layer.forward(inp)
    layer.close()
    ref = moe.moe_forward(inp)
    assert ref["bins"]["counts"].max() > 64
    check(got, ref, "f32")


@pytest.mark.parametrize("layout", [q.QTIP_ACT_ROWS, q.QTIP_ACT_FRAGMENTS])
@pytest.mark.parametrize("variant", [1, 4, 7])
@pytest.mark.parametrize("n", [1, 17, 260])
def test_activation_layouts_full_parity(layout, variant, n):
    """Both activation layouts of the grouped arm (gathered rows; fragment order over 16-padded
    bins with the packing pass), forced on, with experts holding 1, a few and > 64 pairs."""
    inp = moe_inputs.make_inputs(MID, seed=9, n_tokens=n)
    say(f"forward layout={layout} variant={variant} n={n}")
    s = inp.shape
    layer = Layer(inp, arm=q.QTIP_ARM_GROUPED, max_tokens=260)
    q.qtip_moe_plan_destroy(layer.plan)
    layer.plan = q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, 260, q.QTIP_ARM_GROUPED,
                                             variant, q.QTIP_OUT_F32, 0, act_layout=layout), 0)
    import torch
    layer.ws = torch.empty(q.qtip_moe_plan_info(layer.plan)["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
    got = layer.forward(inp)
    layer.close()
    check(got, moe.moe_forward(inp), "f32")
