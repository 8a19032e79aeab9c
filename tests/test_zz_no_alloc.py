"""The allocation-free forward (qtip_moe_forward_noalloc) against qtip_moe_forward.

Both run the same kernels; the allocation-free one keeps its scratch in the library's static
device array, laid out for each call's n.  Two calls in a row, the second with fewer tokens (the
array keeps the first call's contents), must each equal the workspace forward bit for bit, which
is stronger than the parity bar (fp32: max-abs 2e-2 and rel-L2 1e-3; bf16: per element within
2e-2 or one ulp, and rel-L2 1e-3) that is also asserted."""
import numpy as np
import pytest

import moe_inputs
import parity
import trellis_quantized_moe_expert_amd as q
from gpu_util import Layer, say
from moe_inputs.device import tokens_to_device

pytestmark = pytest.mark.gpu


def _noalloc(layer, inp):
    import torch
    t = tokens_to_device(inp)
    n = inp.logits.shape[0]
    dt = torch.float32 if layer.out_dtype == "f32" else torch.int16
    out = torch.full((n, layer.shape.hidden), -1, dtype=dt, device="cuda:0")
    q.qtip_moe_forward_noalloc(layer.plan, layer.w, t.x, t.logits, n, out)
    torch.cuda.synchronize()
    a = out.cpu().numpy()
    return a if layer.out_dtype == "f32" else a.view(np.uint16)


def _same(a, b, out_dtype):
    assert a.shape == b.shape
    if out_dtype == "f32":
        ok, st = parity.check_f32(a, b.astype(np.float64))
    else:
        ok, st = parity.check_bf16(a, b)
    assert ok, st
    assert np.array_equal(a, b), int(np.sum(a != b))


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_tiny_two_calls_second_smaller(out_dtype):
    big = moe_inputs.make_workload("tiny", seed=0)
    small = moe_inputs.redraw_tokens(big, 5, seed=3)
    say(f"noalloc tiny out={out_dtype}: n=16 then n=5")
    layer = Layer(big, out_dtype=out_dtype, max_tokens=16)
    for inp in (big, small):
        _same(_noalloc(layer, inp), layer.forward(inp), out_dtype)
    layer.close()


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_v4_two_calls_second_smaller(out_dtype):
    inps = moe_inputs.make_inputs_multi(moe_inputs.WORKLOADS["v4_decode_n32"], [256, 32, 3], seed=0)
    say(f"noalloc V4 out={out_dtype}: n=256 (grouped), n=32, n=3 (GEMV)")
    layer = Layer(inps[256], out_dtype=out_dtype, max_tokens=1024)
    for n in (256, 32, 3):
        _same(_noalloc(layer, inps[n]), layer.forward(inps[n]), out_dtype)
    layer.close()


def test_lut_rung_v4_two_calls_second_smaller():
    inps = moe_inputs.make_inputs_multi(moe_inputs.WORKLOADS["lut_v4_decode_n32"], [128, 4], seed=0)
    say("noalloc LUT-rung V4: n=128 (grouped), n=4 (GEMV)")
    layer = Layer(inps[128], out_dtype="bf16", max_tokens=1024)
    for n in (128, 4):
        _same(_noalloc(layer, inps[n]), layer.forward(inps[n]), "bf16")
    layer.close()


def test_oversized_call_is_refused_before_any_launch():
    inp = moe_inputs.make_workload("v4_decode_n32", seed=0, n_tokens=8)
    layer = Layer(inp, out_dtype="bf16", max_tokens=1024)
    with pytest.raises(q.QtipError) as ei:
        q.qtip_moe_forward_noalloc(layer.plan, layer.w, 256, 256, 1024, 256)
    assert ei.value.status == q.QTIP_ERR_INVALID_CONFIG and "scratch" in str(ei.value)
    layer.close()
