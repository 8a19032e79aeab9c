"""The arch witness under graph capture, in a fresh process (arch page, "The arch witness").

A process's first call on a device takes the gfx950 witness (a launch and a synchronisation).
If that first call happens while the stream is capturing, the library must decline with
QTIP_ERR_CAPTURING, launch nothing and cache nothing; the same call outside the capture must
then succeed and write every output element.  The check runs in a child process so that no
earlier test has taken the witness already.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, ROOT)
sys.path.insert(0, ROOT + "/tests")
import ctypes
import numpy as np, torch
import moe_inputs
import trellis_quantized_moe_expert_amd as q
from moe_inputs.device import tokens_to_device, weights_to_device
inp = moe_inputs.make_workload("tiny", seed=0)
s = inp.shape
plan = q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, s.n_tokens), 0)
ws = torch.empty(q.qtip_moe_plan_info(plan)["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
d = weights_to_device(inp)
w = q.make_weights(d.codes_gate, d.codes_up, d.codes_down, d.scale_gate, d.scale_up, d.scale_down, d.lut)
t = tokens_to_device(inp)
out = torch.full((s.n_tokens, s.hidden), float("nan"), dtype=torch.float32, device="cuda:0")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
stream = torch.cuda.Stream()
status = None
with torch.cuda.stream(stream):
    g.capture_begin()
    status = q.lib().qtip_moe_forward(plan, ctypes.byref(w), t.x.data_ptr(), t.logits.data_ptr(), s.n_tokens,
                                      out.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream)
    g.capture_end()
torch.cuda.synchronize()
assert status == q.QTIP_ERR_CAPTURING, status
assert q.qtip_moe_stats(plan)["forward_calls"] == 0
q.qtip_moe_forward(plan, w, t.x, t.logits, s.n_tokens, out, ws, ws.numel())
torch.cuda.synchronize()
assert torch.isfinite(out).all().item()
print("witness-capture-ok", flush=True)
"""


def test_first_call_under_capture_is_declined_then_succeeds():
    code = "ROOT = " + repr(ROOT) + "\n" + CHILD
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "witness-capture-ok" in r.stdout
