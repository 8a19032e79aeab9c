"""Degenerate and extreme layer shapes on the GPU, against the declared-mode oracle.

The method's degenerate cases: one expert taking every pair (softmax of one logit is 1, and
its bin spans many 64-pair units); every token routed to every expert (k = E); the largest
router the library accepts (E = 1024, k = 32); the smallest rows (H = I = 128, a single
128-input block whose look-ahead wraps within the same block); a batch much larger than the
experts (thousands of pairs per expert).  Each runs on every arm and, for the grouped arm,
both activation layouts.  Bar: fp32 outputs max-abs 2e-2 and rel-L2 1e-3.
"""
import numpy as np
import pytest

import moe_inputs
import parity
import trellis_quantized_moe_expert_amd as q
from gpu_util import Layer, say
from oracle import moe

pytestmark = pytest.mark.gpu

SHAPES = {
    "one_expert": (moe_inputs.MoEShape(num_experts=1, top_k=1, hidden=256, inter=128, n_tokens=300), 300),
    "k_equals_E": (moe_inputs.MoEShape(num_experts=4, top_k=4, hidden=128, inter=128, n_tokens=50), 50),
    "max_router": (moe_inputs.MoEShape(num_experts=1024, top_k=32, hidden=128, inter=256, n_tokens=40), 40),
    "large_batch": (moe_inputs.MoEShape(num_experts=8, top_k=2, hidden=256, inter=128, n_tokens=2048), 2048),
}

CASES = [(name, arm, layout) for name in SHAPES
         for arm, layout in [(q.QTIP_ARM_GEMV, q.QTIP_ACT_AUTO), (q.QTIP_ARM_GROUPED, q.QTIP_ACT_ROWS),
                             (q.QTIP_ARM_GROUPED, q.QTIP_ACT_FRAGMENTS), (q.QTIP_ARM_DEQUANT, q.QTIP_ACT_AUTO)]]


@pytest.mark.parametrize("name,arm,layout", CASES)
def test_degenerate_and_extreme_shapes(name, arm, layout):
    import torch
    shape, n = SHAPES[name]
    inp = moe_inputs.make_inputs(shape, seed=11, n_tokens=n)
    say(f"edge {name} n={n} arm={arm} layout={layout}")
    s = inp.shape
    layer = Layer(inp, arm=arm, max_tokens=n)
    q.qtip_moe_plan_destroy(layer.plan)
    layer.plan = q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, n, arm, 0, q.QTIP_OUT_F32, 0,
                                             act_layout=layout), 0)
    layer.ws = torch.empty(q.qtip_moe_plan_info(layer.plan)["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    assert st["last_arm"] == arm
    ref = moe.moe_forward(inp)
    if name == "one_expert":
        assert np.allclose(ref["topk_w"], 1.0) and ref["bins"]["counts"][0] == n
    if name == "k_equals_E":
        assert np.all(np.sort(ref["topk_idx"], axis=1) == np.arange(4))
    ok, stats = parity.check_f32(got, ref["out_f64"])
    say(f"  {stats}")
    assert ok, stats
