"""Copy seeded inputs to GPU memory as torch tensors (raw bit patterns, no arithmetic)."""
from __future__ import annotations

import types

import numpy as np


def _t(torch, a: np.ndarray, device):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16 or a.dtype == np.float16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def weights_to_device(inp, device="cuda:0"):
    import torch
    return types.SimpleNamespace(
        codes_gate=_t(torch, inp.codes_gate, device), codes_up=_t(torch, inp.codes_up, device),
        codes_down=_t(torch, inp.codes_down, device), scale_gate=_t(torch, inp.scale_gate, device),
        scale_up=_t(torch, inp.scale_up, device), scale_down=_t(torch, inp.scale_down, device),
        lut=_t(torch, inp.lut, device))


def tokens_to_device(inp, device="cuda:0"):
    import torch
    return types.SimpleNamespace(x=_t(torch, inp.x_bf16, device), logits=_t(torch, inp.logits, device))
