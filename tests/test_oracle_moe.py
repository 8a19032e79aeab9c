"""Pins for the oracle's MoE layer (gated experts, weighted combine, rounding modes).

Pinned against closed forms (all-zero codes make every weight LUT[0]; one-hot
activations read back one decoded weight column; scaling scale_down by 2 doubles
the output; k = E with equal logits averages all experts), permutation
equivariance, and a separately written dense-dequantised reference that routes by
Python sorting, decodes bit by bit and loops token by token.
"""
import dataclasses

import numpy as np
import pytest

import moe_inputs
from oracle import moe, numerics, trellis

SMALL = moe_inputs.MoEShape(num_experts=4, top_k=2, hidden=64, inter=32, n_tokens=6)


def _small(seed=0, **kw):
    return moe_inputs.make_inputs(dataclasses.replace(SMALL, **kw), seed=seed)


@pytest.mark.parametrize("mode", ["declared", "exact"])
def test_binned_forward_matches_dense_reference(mode):
    inp = _small(seed=1)
    a = moe.moe_forward(inp, mode=mode)["out_f64"]
    b = moe.dense_reference(inp, mode=mode, out_dtype="f32")
    assert np.allclose(a.astype(np.float32), b, rtol=1e-6, atol=1e-7)


def test_binned_forward_matches_dense_reference_tiny_workload():
    inp = moe_inputs.make_workload("tiny", seed=0, n_tokens=4)
    a = moe.moe_forward(inp)["out"]
    b = moe.dense_reference(inp)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7)


def test_all_zero_codes_closed_form():
    inp = _small(seed=2)
    inp = dataclasses.replace(inp, codes_gate=np.zeros_like(inp.codes_gate),
                              codes_up=np.zeros_like(inp.codes_up), codes_down=np.zeros_like(inp.codes_down))
    res = moe.moe_forward(inp)
    L = float(numerics.bf16_round(np.float32(inp.lut[0])))
    x = numerics.bf16_bits_to_f64(inp.x_bf16)
    f = lambda a: np.asarray(a, np.float16).astype(np.float64)
    expect = np.zeros((SMALL.n_tokens, SMALL.hidden))
    for t in range(SMALL.n_tokens):
        S = x[t].sum()
        for j in range(SMALL.top_k):
            e = res["topk_idx"][t, j]
            g = f(inp.scale_gate[e]) * L * S
            u = f(inp.scale_up[e]) * L * S
            h = numerics.bf16_round(g / (1 + np.exp(-g)) * u)
            y = f(inp.scale_down[e]) * L * h.sum()
            expect[t] += float(res["topk_w"][t, j]) * y
    assert np.allclose(res["out_f64"], expect, rtol=1e-12, atol=1e-15)


def test_one_hot_activation_reads_back_decoded_column():
    rng = np.random.default_rng(3)
    rows, cols = 24, 40
    codes = rng.integers(0, 256, size=(rows, cols // 4), dtype=np.uint8)
    lut = rng.standard_normal(65536).astype(np.float16)
    scale = rng.uniform(0.5, 2.0, rows).astype(np.float16)
    wdec = trellis.decode_declared(codes, lut)
    for c0 in (0, 17, cols - 1):
        xr = np.zeros((1, cols)); xr[0, c0] = 1.0
        g = (xr @ wdec.T)[0] * scale.astype(np.float64)
        for r in range(rows):
            s = trellis.window_state_bruteforce(trellis.symbols_bruteforce(codes[r]), c0)
            assert g[r] == float(numerics.bf16_round(np.float32(lut[s]))) * float(scale[r])


def test_token_permutation_equivariance():
    inp = _small(seed=4, n_tokens=9)
    perm = np.random.default_rng(0).permutation(9)
    a = moe.moe_forward(inp)["out_f64"]
    b = moe.moe_forward(dataclasses.replace(inp, x_bf16=inp.x_bf16[perm], logits=inp.logits[perm]))["out_f64"]
    assert np.allclose(a[perm], b, rtol=1e-12, atol=1e-15)


def test_scale_down_times_two_doubles_output():
    inp = _small(seed=5)
    a = moe.moe_forward(inp)["out_f64"]
    b = moe.moe_forward(dataclasses.replace(inp, scale_down=(inp.scale_down.astype(np.float32) * 2).astype(np.float16)))["out_f64"]
    assert np.array_equal(2 * a, b)


def test_k_equals_E_equal_logits_averages_experts():
    inp = _small(seed=6, top_k=4)
    inp = dataclasses.replace(inp, logits=np.zeros_like(inp.logits))
    res = moe.moe_forward(inp)
    for t in range(SMALL.n_tokens):
        mean = sum(res["y"][t * 4 + j] for j in range(4)) / 4
        assert np.allclose(res["out_f64"][t], mean, rtol=1e-7, atol=1e-12)


def test_token_subset_equals_full_rows():
    inp = _small(seed=7, n_tokens=10)
    full = moe.moe_forward(inp)["out_f64"]
    sub = moe.moe_forward(inp, tokens=[7, 2, 9])["out_f64"]
    assert np.array_equal(sub, full[[7, 2, 9]])


def test_bf16_output_is_rounded_f32_output():
    inp = _small(seed=8)
    r = moe.moe_forward(inp, out_dtype="bf16")
    assert np.array_equal(r["out"], numerics.f64_to_bf16_bits(r["out_f64"]))


def test_declared_vs_exact_differ_by_bf16_scale_only():
    inp = _small(seed=9, hidden=256, inter=128, n_tokens=8)
    a = moe.moe_forward(inp, mode="declared")["out_f64"]
    b = moe.moe_forward(inp, mode="exact")["out_f64"]
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 1e-4 < rel < 2e-2          # bf16 weights and h: a few 1e-3, not zero, not O(1)
