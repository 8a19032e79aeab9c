"""Pins for the oracle's router logits (hidden states -> one logit per expert).

The router is the plain product logits = x W^T over bf16 operands (the 794-ms-decode-
step page, PR #202, closing list of remaining un-owned items, item (3)).  It is pinned
by a hand-computed example with known bf16 bit patterns (catches a transposed
operand, a dropped term and a wrong bf16 decoding), one-hot rows (exact column
selection), Python-loop brute force on tiny inputs, exact power-of-two scaling, and
a check that an fp32 sequential sum stays inside the stated error bound.
"""
import numpy as np
import pytest

from moe_inputs import MoEShape, f32_to_bf16_bits, make_inputs, make_router_weight
from oracle import router, routing

ONE, TWO, HALF, QUARTER, FOUR = 0x3F80, 0x4000, 0x3F00, 0x3E80, 0x4080
NEG_ONE, NEG_HALF, ZERO = 0xBF80, 0xBF00, 0x0000


def test_hand_example():
    # x = [1, 2, -0.5];  w rows: [1, 0, 0], [0.5, 0.25, 4], [-1, 1, 2]
    x = np.array([[ONE, TWO, NEG_HALF]], np.uint16)
    w = np.array([[ONE, ZERO, ZERO], [HALF, QUARTER, FOUR], [NEG_ONE, ONE, TWO]], np.uint16)
    got = router.router_logits(x, w)
    assert got.shape == (1, 3)
    assert np.array_equal(got, [[1.0, 0.5 + 0.5 - 2.0, -1.0 + 2.0 - 1.0]])


def test_two_tokens_non_square():
    # 2 tokens x 3 inputs, 4 experts: a transposed operand cannot even produce this shape
    x = np.array([[ONE, ZERO, TWO], [ZERO, NEG_ONE, ZERO]], np.uint16)
    w = np.array([[ONE, ONE, ONE], [ZERO, TWO, ZERO], [FOUR, ZERO, HALF], [NEG_HALF, ZERO, ZERO]], np.uint16)
    got = router.router_logits(x, w)
    assert np.array_equal(got, [[3.0, 0.0, 5.0, -0.5], [-1.0, -2.0, 0.0, 0.0]])


def test_one_hot_rows_select_a_column():
    rng = np.random.default_rng(0)
    E, H = 7, 40
    w = f32_to_bf16_bits(rng.standard_normal((E, H)).astype(np.float32))
    x = np.zeros((H, H), np.uint16)
    x[np.arange(H), np.arange(H)] = ONE
    got = router.router_logits(x, w)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, wf.T)


def test_matches_bruteforce():
    rng = np.random.default_rng(1)
    x = f32_to_bf16_bits(rng.standard_normal((3, 11)).astype(np.float32))
    w = f32_to_bf16_bits(rng.standard_normal((5, 11)).astype(np.float32))
    assert np.allclose(router.router_logits(x, w), router.router_logits_bruteforce(x, w), rtol=0, atol=1e-12)


def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(2)
    x = f32_to_bf16_bits(rng.standard_normal((4, 64)).astype(np.float32))
    w = f32_to_bf16_bits(rng.standard_normal((6, 64)).astype(np.float32))
    x2 = (x.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # exponent + 1: every value doubled
    assert np.array_equal(router.router_logits(x2, w), 2.0 * router.router_logits(x, w))


def test_fp32_sum_lies_within_the_bound():
    rng = np.random.default_rng(3)
    H = 4096
    x = f32_to_bf16_bits(rng.standard_normal((8, H)).astype(np.float32))
    w = f32_to_bf16_bits((rng.standard_normal((16, H)) / 64).astype(np.float32))
    exact = router.router_logits(x, w)
    bound = router.router_logits_bound(x, w)
    X = (x.astype(np.uint32) << 16).view(np.float32)
    W = (w.astype(np.uint32) << 16).view(np.float32)
    prod = X[:, None, :] * W[None, :, :]          # exact in fp32
    seq = np.zeros(prod.shape[:2], np.float32)
    for h in range(H):                             # one fp32 rounding per addition
        seq = seq + prod[:, :, h]
    assert np.all(np.abs(seq.astype(np.float64) - exact) <= bound)
    assert np.all(bound <= 1e-3 * np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T + 1e-30)


def test_generated_router_gives_unit_scale_logits():
    s = MoEShape(256, 6, 4096, 2048, 64)
    inp = make_inputs(s, seed=0)
    w = make_router_weight(s, seed=0)
    L = router.router_logits(inp.x_bf16, w)
    assert 0.8 < L.std() < 1.2 and abs(L.mean()) < 0.1


def test_identity_router_routes_on_the_first_features():
    s = MoEShape(8, 2, 256, 128, 16)
    inp = make_inputs(s, seed=1)
    w = np.zeros((8, 256), np.uint16)
    w[np.arange(8), np.arange(8)] = ONE
    idx, _ = routing.route_topk(router.router_logits(inp.x_bf16, w).astype(np.float32), 2)
    xf = (inp.x_bf16[:, :8].astype(np.uint32) << 16).view(np.float32)
    idx2, _ = routing.route_topk(xf, 2)
    assert np.array_equal(idx, idx2)
    out = router.moe_forward_from_hidden(inp, w, out_dtype="f32")
    assert out["out"].shape == (16, 256)


def test_shape_mismatch_is_an_error():
    with pytest.raises(ValueError):
        router.router_logits(np.zeros((2, 3), np.uint16), np.zeros((4, 5), np.uint16))
