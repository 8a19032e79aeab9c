"""Router logits from hidden states, oracle side (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; the product path never calls it.

Source: the 794-ms-decode-step page (PR #202 "The 794 ms decode step, itemised"),
closing list of remaining un-owned items, item (3): the MoE router GEMM, which
turns each token's hidden state into one logit per expert, ran in FP32 on scalar
cores after a cast of the activations; the proposed fix runs it on the matrix
units from bf16 operands.

Reading where the pages are silent: the router weight is one bf16 row of H inputs
per expert, logits[t, e] = sum_h x[t, h] * w[e, h] with no bias, and the logits
are what the top-k routing of the layer consumes.  Both operands are bf16, so
every product is exact in float64 and the oracle's only rounding is the float64
summation; `router_logits_bound` gives the bound any fp32 evaluation of the same
sum (in any order) must meet.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import moe
from .numerics import bf16_bits_to_f64


def router_logits(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * w[e, h] in float64 (x: [n, H], w: [E, H] bf16 bits)."""
    X = bf16_bits_to_f64(x_bits)
    W = bf16_bits_to_f64(w_bits)
    if X.shape[1] != W.shape[1]:
        raise ValueError("x and w must have the same number of inputs")
    return X @ W.T


def router_logits_bruteforce(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """The same sum written as Python loops over scalars (for tiny inputs only)."""
    X = bf16_bits_to_f64(x_bits)
    W = bf16_bits_to_f64(w_bits)
    n, H = X.shape
    E = W.shape[0]
    out = np.zeros((n, E))
    for t in range(n):
        for e in range(E):
            acc = 0.0
            for h in range(H):
                acc += float(X[t, h]) * float(W[e, h])
            out[t, e] = acc
    return out


def router_logits_bound(x_bits: np.ndarray, w_bits: np.ndarray, unit_roundoff: float = 2.0 ** -24) -> np.ndarray:
    """Error bound of an fp32 evaluation of the logits with H additions per logit.

    Each product of two bf16 values is exact in fp32 (8 + 8 significand bits); summing
    H terms in any order with at most one rounding per addition errs by at most
    H * u * sum_h |x w| (first-order bound).  A factor of 2 covers rounding modes
    that may err by a whole unit (truncation) instead of half.
    """
    X = np.abs(bf16_bits_to_f64(x_bits))
    W = np.abs(bf16_bits_to_f64(w_bits))
    H = X.shape[1]
    return 2.0 * H * unit_roundoff * (X @ W.T)


def moe_forward_from_hidden(inp, w_bits: np.ndarray, **kw):
    """The layer with logits computed by `router_logits` (rounded to fp32) from inp.x_bf16."""
    logits = router_logits(inp.x_bf16, w_bits).astype(np.float32)
    return moe.moe_forward(dataclasses.replace(inp, logits=logits), **kw)
