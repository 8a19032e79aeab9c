"""One MoE layer over trellis-coded experts, oracle side (test infrastructure only).

What the layer computes (sources):
* Experts are gate/up/down matrices (workload definition); the pages are silent on
  the activation, so the standard gated expert is read:  h = silu(x W_gate^T) *
  (x W_up^T),  y = h W_down^T,  silu(z) = z / (1 + exp(-z)).
* Each (token, expert) pair's output is weighted by its router weight and summed
  over the token's k choices (the expert forward of the 794-ms-step page, PR #202,
  section "Ruled out by reading", does this with a per-expert gather and
  scatter-add); the sum runs over j = 0..k-1 in ascending order.
* Pairs are processed expert by expert in binned order (gate-the-grouped-GEMM page,
  PR #167, section "The cause is a threshold").

Two evaluation modes:
* "declared": the GPU path's stated rounding points.  x is bf16 (input); the LUT
  value of each weight is narrowed to bf16; the dot product is accumulated wide and
  multiplied by the row's fp16 scale afterwards; h is narrowed to bf16 before the
  down matmul; y and the combine stay wide until the final output cast (bf16
  nearest-even or fp32).  The oracle evaluates everything else in float64.
* "exact": no narrowing anywhere: weights are float32(LUT) * float32(scale), all in
  float64, only the final cast.

`dense_reference` is written separately (textbook per-token loop over
materialised dense weights) to cross-check `moe_forward`.
"""
from __future__ import annotations

import numpy as np

from . import lut_rung, routing, trellis
from .numerics import bf16_bits_to_f64, bf16_round, f64_to_bf16_bits


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def _f16(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).astype(np.float64)


def expert_declared(xr, wg, wu, wd, sg, su, sd):
    """Gated expert on rows xr with unscaled bf16 weights; scales after each dot product."""
    g = (xr @ wg.T) * _f16(sg)[None, :]
    u = (xr @ wu.T) * _f16(su)[None, :]
    h = bf16_round(silu(g) * u)
    y = (h @ wd.T) * _f16(sd)[None, :]
    return y, h


def expert_exact(xr, wg, wu, wd):
    """Gated expert with scaled float weights, no intermediate narrowing."""
    h = silu(xr @ wg.T) * (xr @ wu.T)
    return h @ wd.T, h


def _finish(acc: np.ndarray, out_dtype: str) -> np.ndarray:
    if out_dtype == "f32":
        return acc.astype(np.float32)
    if out_dtype == "bf16":
        return f64_to_bf16_bits(acc)
    raise ValueError(out_dtype)


def _decoder(inp):
    """The decode of the layer's rung: the bitshift rung's 16-bit-window LUT (oracle.trellis) or
    the LUT rung's 2-D codebook (oracle.lut_rung)."""
    rung = getattr(inp.shape, "rung", "bitshift")
    if rung == "bitshift":
        return trellis
    if rung == "lut":
        return lut_rung
    raise ValueError(rung)


def decode_expert(inp, e: int, mode: str = "declared"):
    """Expert e's gate, up and down weights: unscaled bf16 table values in declared mode (the
    scales are applied after each dot product), float32(table) * float32(scale) in exact mode."""
    dec = _decoder(inp)
    if mode == "declared":
        return tuple(dec.decode_declared(dec.stored_rows(c[e]), inp.lut)
                     for c in (inp.codes_gate, inp.codes_up, inp.codes_down))
    if mode == "exact":
        return tuple(dec.decode_exact(dec.stored_rows(c[e]), inp.lut, sc[e])
                     for c, sc in ((inp.codes_gate, inp.scale_gate), (inp.codes_up, inp.scale_up),
                                   (inp.codes_down, inp.scale_down)))
    raise ValueError(mode)


def expert_pairs(inp, e: int, pids, mode: str = "declared", weights=None):
    """Outputs y [len(pids), H] and intermediates h of expert e for the binned pairs `pids`
    (pair id p = t*k + j reads token t = p // k).  `weights`, if given, is
    decode_expert(inp, e, mode), so one decode can serve several calls."""
    k = inp.shape.top_k
    pids = np.asarray(pids, np.int64)
    xr = bf16_bits_to_f64(inp.x_bf16[pids // k])
    wg, wu, wd = weights if weights is not None else decode_expert(inp, e, mode)
    if mode == "declared":
        return expert_declared(xr, wg, wu, wd, inp.scale_gate[e], inp.scale_up[e], inp.scale_down[e])
    if mode == "exact":
        return expert_exact(xr, wg, wu, wd)
    raise ValueError(mode)


def combine(y: dict, topk_w: np.ndarray, tokens, k: int, hidden: int) -> np.ndarray:
    """out[t] = sum_{j=0..k-1} w[t, j] * y[t*k + j], j ascending (float64), for each token listed."""
    acc = np.zeros((len(tokens), hidden), np.float64)
    for r, t in enumerate(tokens):
        for j in range(k):
            acc[r] += np.float64(topk_w[t, j]) * y[t * k + j]
    return acc


def finish(acc: np.ndarray, out_dtype: str) -> np.ndarray:
    """The single final cast: fp32 values, or bf16 bit patterns (via fp32, nearest-even)."""
    return _finish(acc, out_dtype)


def moe_forward(inp, tile_m: int = 16, mode: str = "declared", out_dtype: str = "f32",
                tokens=None) -> dict:
    """Route, bin, run each woken expert over its binned pairs, combine.

    `inp` carries lut, codes_*, scale_*, x_bf16, logits and shape (moe_inputs.MoEInputs).
    `tokens`: optional list of token indices; only the pairs of those tokens are
    evaluated and `out` holds their rows in that order (the routing and binning
    are still computed for the whole batch).
    """
    s = inp.shape
    E, k, H = s.num_experts, s.top_k, s.hidden
    n = inp.logits.shape[0]
    idx, w = routing.route_topk(inp.logits, k)
    bins = routing.bin_pairs(idx, E, tile_m)
    want = None if tokens is None else set(int(t) for t in tokens)
    y = {}
    h_sorted = {}
    for e in range(E):
        start, cnt = int(bins["offsets"][e]), int(bins["counts"][e])
        pids = bins["sorted_pair"][start:start + cnt]
        if want is not None:
            pids = np.array([p for p in pids if int(p) // k in want], np.int32)
        if len(pids) == 0:
            continue
        ye, he = expert_pairs(inp, e, pids, mode)
        for q, p in enumerate(pids):
            y[int(p)] = ye[q]
            h_sorted[int(p)] = he[q]
    toks = list(range(n)) if tokens is None else [int(t) for t in tokens]
    acc = combine(y, w, toks, k, H)
    return {"out": _finish(acc, out_dtype), "out_f64": acc, "topk_idx": idx, "topk_w": w,
            "bins": bins, "y": y, "h": h_sorted}


def dense_reference(inp, mode: str = "declared", out_dtype: str = "f32") -> np.ndarray:
    """Textbook MoE forward over weights materialised element by element.

    Routing by Python sorting, weights by the bit-by-bit decoder, then a plain loop
    over tokens and their k experts (no binning).  Pure Python decode: tiny shapes only.
    """
    s = inp.shape
    E, k, H = s.num_experts, s.top_k, s.hidden
    idx, w = routing.route_topk_bruteforce(inp.logits, k)
    declared = mode == "declared"
    dense = {}
    n = inp.logits.shape[0]
    out = np.zeros((n, H), np.float64)
    for t in range(n):
        xr = bf16_bits_to_f64(inp.x_bf16[t])
        for j in range(k):
            e = int(idx[t, j])
            if e not in dense:
                dec = _decoder(inp)
                dense[e] = [dec.dense_weights_bruteforce(dec.stored_rows(c[e]), inp.lut, sc[e], declared)
                            for c, sc in ((inp.codes_gate, inp.scale_gate), (inp.codes_up, inp.scale_up),
                                          (inp.codes_down, inp.scale_down))]
            wg, wu, wd = dense[e]
            if declared:
                g = np.array([float(np.dot(xr, wg[r])) for r in range(wg.shape[0])]) * _f16(inp.scale_gate[e])
                u = np.array([float(np.dot(xr, wu[r])) for r in range(wu.shape[0])]) * _f16(inp.scale_up[e])
                h = bf16_round(g / (1.0 + np.exp(-g)) * u)
                yv = np.array([float(np.dot(h, wd[r])) for r in range(wd.shape[0])]) * _f16(inp.scale_down[e])
            else:
                g = wg @ xr
                u = wu @ xr
                h = g / (1.0 + np.exp(-g)) * u
                yv = wd @ h
            out[t] += np.float64(w[t, j]) * yv
    return _finish(out, out_dtype)
