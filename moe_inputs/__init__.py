"""Seeded synthetic inputs for one MoE layer with 2-bit bitshift-trellis expert weights.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no decoding, routing, matmul or rounding of results).  Both
the CPU oracle's tests and the GPU path's tests and benchmark take their inputs
from here, so neither side depends on the other to produce data.

Shapes follow the trellis-MoE workloads: E experts, top-k routing, hidden size H,
expert intermediate size I, n tokens.  Every expert has three matrices (gate and
up of shape [I, H], down of shape [H, I]); a matrix with `rows` outputs and `cols`
inputs is stored as `rows * cols / 4` bytes of packed 2-bit codes (uniform random
bits) plus one fp16 scale per output row drawn from U(0.01, 0.05).  One shared
65536-entry fp16 lookup table holds N(0,1) samples.  Activations are N(0,1)
rounded to bf16; router logits are N(0,1) float32, or, for the skewed-router
workload, log-popularity under a Zipf(s) law plus Gumbel(0,1) noise.

Draw order from one numpy PCG64 generator is fixed: the LUT, then for each expert
e = 0..E-1 the gate codes, gate scales, up codes, up scales, down codes, down
scales, then the activations, then the logits.  The arrays are plain numpy arrays;
bf16 values are carried as their uint16 bit patterns.

For layers that start from hidden states, a router weight [E, H] of N(0, 1/H)
samples rounded to bf16 comes from a second generator, PCG64([seed, 1]), so the
draws above do not change; with N(0,1) activations its logits are close to N(0,1).

Layers of the LUT rung (shape.rung == "lut") draw, in the LUT's place, a codebook of
2**9 two-dimensional fp16 N(0,1) samples ([512, 2], carried in the `lut` field); the
codes, scales, activations and logits are drawn exactly as for the bitshift rung.  Code bytes
are uniform random, so their storage order (block-interleaved, as the kernels and the oracle
read them) does not change what is drawn.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

LUT_SIZE = 65536


@dataclasses.dataclass
class MoEShape:
    num_experts: int
    top_k: int
    hidden: int
    inter: int
    n_tokens: int
    routing: str = "uniform"      # "uniform" (logits N(0,1)) or "zipf"
    zipf_s: float = 1.1
    rung: str = "bitshift"        # "bitshift" (65536-entry LUT) or "lut" (512 x 2 codebook)


@dataclasses.dataclass
class MoEInputs:
    shape: MoEShape
    seed: int
    lut: np.ndarray          # [65536] float16 (bitshift rung) or [512, 2] float16 codebook (LUT rung)
    codes_gate: np.ndarray   # [E, I, H/4] uint8
    codes_up: np.ndarray     # [E, I, H/4] uint8
    codes_down: np.ndarray   # [E, H, I/4] uint8
    scale_gate: np.ndarray   # [E, I] float16
    scale_up: np.ndarray     # [E, I] float16
    scale_down: np.ndarray   # [E, H] float16
    x_bf16: np.ndarray       # [n, H] uint16 (bf16 bit patterns)
    logits: np.ndarray       # [n, E] float32


# The workloads the method is measured on (trellis MoE layer shapes).
WORKLOADS = {
    "tiny": MoEShape(8, 2, 256, 128, 16),
    "v4_decode_n32": MoEShape(256, 6, 4096, 2048, 32),
    "v4_mid_n128": MoEShape(256, 6, 4096, 2048, 128),
    "v4_mid_n512": MoEShape(256, 6, 4096, 2048, 512),
    "v4_full_n683": MoEShape(256, 6, 4096, 2048, 683),
    "v4_full_n1024": MoEShape(256, 6, 4096, 2048, 1024),
    "v4_zipf_n256": MoEShape(256, 6, 4096, 2048, 256, routing="zipf", zipf_s=1.1),
    # a one-token decode step of the same layer: the low-fill extreme, reported beside the others
    "v4_decode_n1": MoEShape(256, 6, 4096, 2048, 1),
    # the same layers with LUT-rung experts (a 512 x 2 codebook instead of the 65536-entry LUT)
    "lut_tiny": MoEShape(8, 2, 256, 128, 16, rung="lut"),
    "lut_v4_decode_n1": MoEShape(256, 6, 4096, 2048, 1, rung="lut"),
    "lut_v4_decode_n32": MoEShape(256, 6, 4096, 2048, 32, rung="lut"),
    "lut_v4_mid_n128": MoEShape(256, 6, 4096, 2048, 128, rung="lut"),
    "lut_v4_mid_n512": MoEShape(256, 6, 4096, 2048, 512, rung="lut"),
    "lut_v4_full_n1024": MoEShape(256, 6, 4096, 2048, 1024, rung="lut"),
    "lut_v4_zipf_n256": MoEShape(256, 6, 4096, 2048, 256, routing="zipf", zipf_s=1.1, rung="lut"),
}

LUT_RUNG_BITS = 9   # codebook index bits of the LUT rung (2**9 entries of two fp16 values)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Used only to produce bf16 input activations.  Inputs are finite samples.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def _draw_experts(rng: np.random.Generator, s: MoEShape):
    E, H, I = s.num_experts, s.hidden, s.inter
    cg = np.empty((E, I, H // 4), np.uint8)
    cu = np.empty((E, I, H // 4), np.uint8)
    cd = np.empty((E, H, I // 4), np.uint8)
    sg = np.empty((E, I), np.float16)
    su = np.empty((E, I), np.float16)
    sd = np.empty((E, H), np.float16)
    for e in range(E):
        cg[e] = rng.integers(0, 256, size=(I, H // 4), dtype=np.uint8)
        sg[e] = rng.uniform(0.01, 0.05, size=I).astype(np.float16)
        cu[e] = rng.integers(0, 256, size=(I, H // 4), dtype=np.uint8)
        su[e] = rng.uniform(0.01, 0.05, size=I).astype(np.float16)
        cd[e] = rng.integers(0, 256, size=(H, I // 4), dtype=np.uint8)
        sd[e] = rng.uniform(0.01, 0.05, size=H).astype(np.float16)
    return cg, cu, cd, sg, su, sd


def _draw_table(rng: np.random.Generator, s: MoEShape) -> np.ndarray:
    if s.rung == "bitshift":
        return rng.standard_normal(LUT_SIZE).astype(np.float16)
    if s.rung == "lut":
        return rng.standard_normal((1 << LUT_RUNG_BITS, 2)).astype(np.float16)
    raise ValueError(f"unknown rung {s.rung!r}")


def _draw_logits(rng: np.random.Generator, s: MoEShape) -> np.ndarray:
    n, E = s.n_tokens, s.num_experts
    if s.routing == "uniform":
        return rng.standard_normal((n, E)).astype(np.float32)
    if s.routing == "zipf":
        # Popularity p_e proportional to rank_e^-s over a seeded random ranking; adding
        # Gumbel(0,1) noise to log p_e makes the top-k a draw of k distinct experts
        # without replacement in proportion to p.
        ranks = rng.permutation(E) + 1
        logp = -s.zipf_s * np.log(ranks.astype(np.float64))
        logp -= np.log(np.exp(logp).sum())
        g = rng.gumbel(0.0, 1.0, size=(n, E))
        return (logp[None, :] + g).astype(np.float32)
    raise ValueError(f"unknown routing {s.routing!r}")


def make_inputs(shape: MoEShape, seed: int = 0, n_tokens: Optional[int] = None) -> MoEInputs:
    """Draw one MoE layer's weights and one batch of activations/logits."""
    s = dataclasses.replace(shape, n_tokens=shape.n_tokens if n_tokens is None else n_tokens)
    if s.hidden % 4 or s.inter % 4:
        raise ValueError("hidden and inter must be multiples of 4 (4 symbols per byte)")
    rng = np.random.Generator(np.random.PCG64(seed))
    lut = _draw_table(rng, s)
    cg, cu, cd, sg, su, sd = _draw_experts(rng, s)
    x = f32_to_bf16_bits(rng.standard_normal((s.n_tokens, s.hidden)).astype(np.float32))
    logits = _draw_logits(rng, s)
    return MoEInputs(s, seed, lut, cg, cu, cd, sg, su, sd, x, logits)


def make_inputs_multi(shape: MoEShape, n_list, seed: int = 0) -> dict:
    """One set of weights and, for each n in n_list, the activations and logits that
    make_inputs(shape, seed, n) would draw (the generator state after the weights is
    replayed for each n).  Returns {n: MoEInputs}, all sharing the weight arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lut = _draw_table(rng, shape)
    weights = _draw_experts(rng, shape)
    state = rng.bit_generator.state
    out = {}
    for n in n_list:
        s = dataclasses.replace(shape, n_tokens=n)
        r = np.random.Generator(np.random.PCG64(seed))
        r.bit_generator.state = state
        x = f32_to_bf16_bits(r.standard_normal((n, s.hidden)).astype(np.float32))
        out[n] = MoEInputs(s, seed, lut, *weights, x, _draw_logits(r, s))
    return out


def make_router_weight(shape: MoEShape, seed: int = 0) -> np.ndarray:
    """Router weight [E, H] as bf16 bit patterns: N(0, 1/H) samples from PCG64([seed, 1])."""
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    w = rng.standard_normal((shape.num_experts, shape.hidden)) / np.sqrt(shape.hidden)
    return f32_to_bf16_bits(w.astype(np.float32))


def make_workload(name: str, seed: int = 0, n_tokens: Optional[int] = None) -> MoEInputs:
    return make_inputs(WORKLOADS[name], seed=seed, n_tokens=n_tokens)


def draw_logits(shape: MoEShape, seed: int = 0) -> np.ndarray:
    """Router logits alone (own stream), for routing-only tests at the workload's sizes."""
    rng = np.random.Generator(np.random.PCG64([seed, 0x10617]))
    return _draw_logits(rng, shape)


def redraw_tokens(inp: MoEInputs, n_tokens: int, seed: int) -> MoEInputs:
    """Keep the weights, draw a fresh batch of n_tokens activations and logits."""
    s = dataclasses.replace(inp.shape, n_tokens=n_tokens)
    rng = np.random.Generator(np.random.PCG64([seed, 0x70CE]))
    x = f32_to_bf16_bits(rng.standard_normal((n_tokens, s.hidden)).astype(np.float32))
    logits = _draw_logits(rng, s)
    return dataclasses.replace(inp, shape=s, x_bf16=x, logits=logits)
