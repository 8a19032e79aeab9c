"""Router GEMM on the GPU (qtip_moe_router_logits, qtip_moe_forward_hidden) vs the oracle.

Bars:
* logits: every element within the fp32 summation bound of the oracle's float64 value,
  2 H 2^-24 sum_h |x w| (bf16 products are exact in fp32; one rounding per addition);
* the layer from hidden states equals the layer from the library's own router logits bit
  for bit (one computation, two entry points);
* routing from hidden states is, for every token, a valid top-k of some logits within the
  bound of the oracle's, and equals the oracle's routing (on its float64 logits rounded to
  fp32) wherever the measured logit deviation cannot reorder the top k; the layer output
  then meets the usual parity bar on those tokens.
Shapes span several 32x32 output tiles with ragged token and expert tails, E not a
multiple of 4, every K split the plan picks, and the full V4 router (E=256, H=4096).
"""
import numpy as np
import pytest

import moe_inputs
import parity
import trellis_quantized_moe_expert_amd as q
from gpu_util import Layer, say
from moe_inputs.device import tokens_to_device
from oracle import router, routing

pytestmark = pytest.mark.gpu

V4 = moe_inputs.WORKLOADS["v4_decode_n32"]
ODD = moe_inputs.MoEShape(num_experts=36, top_k=3, hidden=384, inter=128, n_tokens=50)
TEN = moe_inputs.MoEShape(num_experts=10, top_k=2, hidden=256, inter=128, n_tokens=19)
MID = moe_inputs.MoEShape(num_experts=16, top_k=4, hidden=512, inter=256, n_tokens=100)


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0")


def gpu_logits(layer, x_dev, w_dev, n):
    import torch
    lg = torch.empty((n, layer.shape.num_experts), dtype=torch.float32, device="cuda:0")
    q.qtip_moe_router_logits(layer.plan, x_dev, w_dev, n, lg, layer.ws, layer.ws.numel())
    torch.cuda.synchronize()
    return lg.cpu().numpy()


CASES = [("tiny", moe_inputs.WORKLOADS["tiny"], 16), ("ten", TEN, 19), ("odd", ODD, 50), ("odd", ODD, 1),
         ("mid", MID, 1), ("mid", MID, 9), ("mid", MID, 100), ("mid", MID, 300),
         ("v4", V4, 1), ("v4", V4, 32), ("v4", V4, 683), ("v4", V4, 1024)]


@pytest.mark.parametrize("name,shape,n", CASES)
def test_router_logits_within_the_fp32_bound(name, shape, n):
    inp = moe_inputs.make_inputs(shape, seed=4, n_tokens=n)
    w = moe_inputs.make_router_weight(shape, seed=4)
    layer = Layer(inp, max_tokens=max(n, 300 if name == "mid" else n))
    S = q.qtip_moe_router_split(layer.plan, n)
    say(f"router logits {name} n={n} E={shape.num_experts} H={shape.hidden} split={S}")
    got = gpu_logits(layer, tokens_to_device(inp).x, to_dev(w), n)
    layer.close()
    ref = router.router_logits(inp.x_bf16, w)
    bound = router.router_logits_bound(inp.x_bf16, w)
    err = np.abs(got.astype(np.float64) - ref)
    say(f"  max err {err.max():.3e}, max bound {bound.max():.3e}")
    assert got.shape == ref.shape and np.all(np.isfinite(got))
    assert np.all(err <= bound), int(np.sum(err > bound))


@pytest.mark.parametrize("name,shape,n", [("tiny", moe_inputs.WORKLOADS["tiny"], 16), ("mid", MID, 100),
                                          ("v4", V4, 32)])
def test_forward_hidden_equals_forward_of_router_logits(name, shape, n):
    import torch
    inp = moe_inputs.make_inputs(shape, seed=5, n_tokens=n)
    w_dev = to_dev(moe_inputs.make_router_weight(shape, seed=5))
    say(f"forward_hidden vs forward(router_logits) {name} n={n}")
    layer = Layer(inp, out_dtype="f32")
    x = tokens_to_device(inp).x
    lg = torch.empty((n, shape.num_experts), dtype=torch.float32, device="cuda:0")
    q.qtip_moe_router_logits(layer.plan, x, w_dev, n, lg, layer.ws, layer.ws.numel())
    out_a = torch.empty((n, shape.hidden), dtype=torch.float32, device="cuda:0")
    q.qtip_moe_forward(layer.plan, layer.w, x, lg, n, out_a, layer.ws, layer.ws.numel())
    q.qtip_moe_stats_reset(layer.plan)
    out_b = torch.empty_like(out_a)
    q.qtip_moe_forward_hidden(layer.plan, layer.w, w_dev, x, n, out_b, layer.ws, layer.ws.numel())
    torch.cuda.synchronize()
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    assert st["router_launches"] == 1 and st["forward_calls"] == 1
    assert np.array_equal(out_a.cpu().numpy().view(np.uint32), out_b.cpu().numpy().view(np.uint32))


def decided_tokens(ref_logits, tol, k):
    """Tokens whose top-k (and its order) survives any change of each logit by up to tol[t]."""
    srt = -np.sort(-ref_logits, axis=1)
    gaps = srt[:, :k] - srt[:, 1:k + 1]
    return np.nonzero(np.all(gaps > 2.0 * tol[:, None], axis=1))[0]


def valid_under_bound(sel, L, B):
    """True if the ordered selection is the top-k of some logits within B of L."""
    lo, hi = L - B, L + B
    for i in range(len(sel) - 1):
        if hi[sel[i]] < lo[sel[i + 1]]:
            return False
    rest = np.setdiff1d(np.arange(len(L)), sel)
    return bool(np.all(lo[rest] <= hi[sel[-1]]))


@pytest.mark.parametrize("name,shape,n,sample", [("mid", MID, 300, None), ("v4", V4, 1024, [0, 511, 1023])])
def test_routing_and_layer_from_hidden_states_match_the_oracle(name, shape, n, sample):
    import torch
    inp = moe_inputs.make_inputs(shape, seed=6, n_tokens=n)
    w = moe_inputs.make_router_weight(shape, seed=6)
    say(f"layer from hidden states {name} n={n}")
    layer = Layer(inp, out_dtype="f32")
    x = tokens_to_device(inp).x
    w_dev = to_dev(w)
    lg = gpu_logits(layer, x, w_dev, n)
    # the library's routing of its own logits, through the routing entry point
    k, E = shape.top_k, shape.num_experts
    lg_dev = torch.from_numpy(lg).to("cuda:0")
    idx = torch.empty((n, k), dtype=torch.int32, device="cuda:0")
    wts = torch.empty((n, k), dtype=torch.float32, device="cuda:0")
    counts = torch.empty(E, dtype=torch.int32, device="cuda:0")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda:0")
    sp = torch.empty(n * k, dtype=torch.int32, device="cuda:0")
    tmap = torch.empty((n * k + E + 1) * 3, dtype=torch.int32, device="cuda:0")
    ntl = torch.empty(1, dtype=torch.int32, device="cuda:0")
    q.qtip_moe_route(layer.plan, lg_dev, n, idx, wts, counts, offs, sp, tmap, ntl)
    out = torch.empty((n, shape.hidden), dtype=torch.float32, device="cuda:0")
    q.qtip_moe_forward_hidden(layer.plan, layer.w, w_dev, x, n, out, layer.ws, layer.ws.numel())
    torch.cuda.synchronize()
    got_idx, got = idx.cpu().numpy(), out.cpu().numpy()
    layer.close()

    ref_lg = router.router_logits(inp.x_bf16, w)
    bound = router.router_logits_bound(inp.x_bf16, w)
    ref_idx, _ = routing.route_topk(ref_lg.astype(np.float32), k)
    # every selection is a valid top-k of logits within the bound of the oracle's
    assert all(valid_under_bound(got_idx[t], ref_lg[t], bound[t]) for t in range(n))
    # where the measured deviation (plus the oracle's own fp32 rounding) cannot reorder the
    # top k, the selection is the oracle's
    dev = np.abs(lg.astype(np.float64) - ref_lg).max(axis=1) + 1e-6 * np.abs(ref_lg).max(axis=1)
    dec = decided_tokens(ref_lg, dev, k)
    say(f"  {len(dec)} of {n} tokens decided beyond the measured deviation (max {dev.max():.2e})")
    assert len(dec) >= 0.98 * n
    assert np.array_equal(got_idx[dec], ref_idx[dec])
    toks = [int(t) for t in (dec if sample is None else sample) if t in set(dec.tolist())]
    assert toks
    ref = router.moe_forward_from_hidden(inp, w, tokens=toks)
    ok, st = parity.check_f32(got[toks], ref["out_f64"])
    say(f"  {st}")
    assert ok, st
