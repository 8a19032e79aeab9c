"""Helpers for GPU tests: run the HIP path through the C ABI on seeded inputs."""
import numpy as np

import trellis_quantized_moe_expert_amd as q
from moe_inputs.device import tokens_to_device, weights_to_device


def say(*a):
    print(*a, flush=True)


def rung_code(shape):
    return q.QTIP_RUNG_LUT if getattr(shape, "rung", "bitshift") == "lut" else q.QTIP_RUNG_BITSHIFT


class Layer:
    """A plan + device weights + workspace for one MoE layer."""

    def __init__(self, inp, arm=q.QTIP_ARM_AUTO, out_dtype="f32", max_tokens=None, tile_m=0, weights=None):
        import torch
        s = inp.shape
        self.shape = s
        self.out_dtype = out_dtype
        od = q.QTIP_OUT_F32 if out_dtype == "f32" else q.QTIP_OUT_BF16
        self.desc = q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, max_tokens or s.n_tokens, arm, 0, od, tile_m,
                                rung=rung_code(s))
        self.plan = q.qtip_moe_plan(self.desc, 0)
        self.info = q.qtip_moe_plan_info(self.plan)
        self.ws = torch.empty(self.info["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
        self.dw = weights if weights is not None else weights_to_device(inp)
        d = self.dw
        self.w = q.make_weights(d.codes_gate, d.codes_up, d.codes_down, d.scale_gate, d.scale_up, d.scale_down, d.lut)

    def forward(self, inp):
        import torch
        t = tokens_to_device(inp)
        n = inp.logits.shape[0]
        dt = torch.float32 if self.out_dtype == "f32" else torch.int16
        out = torch.empty((n, self.shape.hidden), dtype=dt, device="cuda:0")
        q.qtip_moe_forward(self.plan, self.w, t.x, t.logits, n, out, self.ws, self.ws.numel())
        torch.cuda.synchronize()
        a = out.cpu().numpy()
        return a if self.out_dtype == "f32" else a.view(np.uint16)

    def close(self):
        q.qtip_moe_plan_destroy(self.plan)
