"""The layer under HIP graph capture.

The plan is host-only and the dispatch predicate is a closed form in host scalars (m-tile
page, "The fix": safe inside graph capture), so after the first call on a device has taken the
arch witness, a whole forward can be captured and replayed.  Each replay runs after eager
work of the program's own (another forward into another buffer, then a synchronisation) and
must reproduce the eager result bit for bit; inputs changed in place between replays must be
picked up by the replay.
"""
import numpy as np
import pytest

import moe_inputs
import trellis_quantized_moe_expert_amd as q
from gpu_util import Layer, say
from moe_inputs.device import tokens_to_device

pytestmark = pytest.mark.gpu

MID = moe_inputs.MoEShape(num_experts=16, top_k=4, hidden=512, inter=256, n_tokens=100)


def bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("name,shape,n,arm", [("mid", MID, 100, q.QTIP_ARM_GROUPED), ("mid", MID, 6, q.QTIP_ARM_GEMV),
                                              ("mid", MID, 40, q.QTIP_ARM_DEQUANT),
                                              ("v4", moe_inputs.WORKLOADS["v4_decode_n32"], 32, q.QTIP_ARM_AUTO),
                                              ("v4", moe_inputs.WORKLOADS["v4_full_n1024"], 1024, q.QTIP_ARM_AUTO),
                                              ("lut_v4", moe_inputs.WORKLOADS["lut_v4_decode_n32"], 32, q.QTIP_ARM_AUTO),
                                              ("lut_v4", moe_inputs.WORKLOADS["lut_v4_decode_n32"], 3, q.QTIP_ARM_AUTO)])
def test_captured_forward_replays_match_eager(name, shape, n, arm):
    import torch
    inp = moe_inputs.make_inputs(shape, seed=12, n_tokens=n)
    other = moe_inputs.redraw_tokens(inp, n, seed=13)
    say(f"graph capture {name} n={n} arm={arm}")
    layer = Layer(inp, arm=arm, out_dtype="f32", max_tokens=n)
    t, t2 = tokens_to_device(inp), tokens_to_device(other)
    H = shape.hidden
    out_eager = torch.empty((n, H), dtype=torch.float32, device="cuda:0")
    out_other = torch.empty_like(out_eager)
    out_graph = torch.empty_like(out_eager)
    fwd = lambda x, lg, out: q.qtip_moe_forward(layer.plan, layer.w, x, lg, n, out, layer.ws, layer.ws.numel())
    fwd(t.x, t.logits, out_eager)            # also takes the arch witness outside the capture
    fwd(t2.x, t2.logits, out_other)
    torch.cuda.synchronize()
    want, want_other = bits(out_eager), bits(out_other)

    # capture on a side stream with inputs in fixed buffers
    x_buf, lg_buf = t.x.clone(), t.logits.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fwd(x_buf, lg_buf, out_graph)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        out_graph.fill_(float("nan"))
        fwd(t2.x, t2.logits, out_other)      # eager work of the program's own between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_graph), want), f"replay {rep}"
        assert np.array_equal(bits(out_other), want_other)
    # the replay reads its input buffers: other inputs copied in give the other result
    x_buf.copy_(t2.x)
    lg_buf.copy_(t2.logits)
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_graph), want_other)
    layer.close()
