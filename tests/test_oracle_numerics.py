"""Pins of the oracle's bf16 output cast, numerics.f64_to_bf16_bits.

The cast is the last step of every bf16 parity check (the layer output is rounded once,
from the fp32 the path holds, to bf16 nearest-even).  It is pinned against three things
that do not come from the function itself:
  * hand-derived bit patterns of exact ties and near-ties (worked out on paper below);
  * a brute-force nearest-value search over the neighbouring bf16 patterns;
  * torch's own float32 -> bfloat16 conversion over every finite fp16 value and random doubles.
Planted mutations (ties away from zero, truncation, ties toward odd, rounding straight from
float64) must each fail at least one pin.
"""
import numpy as np
import pytest

from oracle import numerics

# (value, expected bf16 bits).  bf16 keeps 7 fraction bits, so near 1.0 its spacing is 2^-7
# and the midpoints are odd multiples of 2^-8.
HAND_CASES = [
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),            # tie between 0x3F80 (even) and 0x3F81: even wins
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie between 0x3F81 (odd) and 0x3F82 (even)
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (-(1.0 + 3 * 2.0 ** -8), 0xBF82),
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie, still visible in float32
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F80),  # lost when rounding to float32 first: a tie again
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),  # just below the tie
    (2.0 + 2.0 ** -7, 0x4000),            # tie at spacing 2^-6: lower neighbour 0x4000 is even
    (2.0 + 3 * 2.0 ** -7, 0x4002),
    (0.1, 0x3DCD),                        # 0.1 = 0x3DCCCCCD in float32, rounds up
    (-3.140625, 0xC049),                  # exactly representable: 0xC049 = -(1 + 73/128) * 2
    (65504.0, 0x4780),                    # largest fp16: 0x477FE000 rounds up to 0x4780
]


def _bits_to_f64(bits):
    return numerics.bf16_bits_to_f64(np.asarray(bits, np.uint16))


def _nearest_bf16_bruteforce(x):
    """For each float32 value, the bf16 pattern among {truncation, its two neighbours} that is
    nearest, ties to the even pattern (checked by direct distance comparison)."""
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32)
    base = (u >> 16).astype(np.int64)
    best = np.zeros(f.shape, np.uint16)
    for i, xv in enumerate(f.astype(np.float64).ravel()):
        b0 = int(base.ravel()[i])
        cands = [c for c in (b0 - 1, b0, b0 + 1) if 0 <= c <= 0xFFFF and (c & 0x7F80) != 0x7F80]
        dist = [(abs(float(_bits_to_f64(c)) - xv), c & 1, c) for c in cands]
        dist.sort()
        best.ravel()[i] = dist[0][2]
    return best


def _pins_hold(fn) -> bool:
    """True when `fn` (float64 array -> bf16 bits) passes every pin of this module."""
    vals = np.array([v for v, _ in HAND_CASES], np.float64)
    exp = np.array([b for _, b in HAND_CASES], np.uint16)
    if not np.array_equal(np.asarray(fn(vals), np.uint16), exp):
        return False
    rng = np.random.Generator(np.random.PCG64(11))
    x = np.concatenate([rng.standard_normal(3000) * 8.0, rng.standard_normal(500) * 1e-3,
                        # exact float32 ties: bit 15 set and the bits below it clear
                        ((rng.integers(0x3000, 0x4800, 500).astype(np.uint32) << 16) | 0x8000)
                        .view(np.float32).astype(np.float64)])
    if not np.array_equal(np.asarray(fn(x), np.uint16), _nearest_bf16_bruteforce(x)):
        return False
    torch = pytest.importorskip("torch")
    allf16 = np.arange(0x10000, dtype=np.uint16).view(np.float16)
    allf16 = allf16[np.isfinite(allf16)].astype(np.float64)
    ref = torch.from_numpy(allf16.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if not np.array_equal(np.asarray(fn(allf16), np.uint16), ref):
        return False
    y = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bool(np.array_equal(np.asarray(fn(y), np.uint16), ref))


def test_f64_to_bf16_bits_passes_every_pin():
    assert _pins_hold(numerics.f64_to_bf16_bits)


def test_hand_cases_one_by_one():
    for v, b in HAND_CASES:
        assert int(numerics.f64_to_bf16_bits(np.array([v]))[0]) == b, (v, hex(b))


def test_bits_and_values_agree_with_bf16_round():
    rng = np.random.Generator(np.random.PCG64(12))
    x = rng.standard_normal(10000) * 5
    assert np.array_equal(_bits_to_f64(numerics.f64_to_bf16_bits(x)), numerics.bf16_round(x))


def _u32(a):
    return np.asarray(a, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)


MUTANTS = {
    "ties away from zero": lambda a: ((_u32(a) + 0x8000) >> 16).astype(np.uint16),
    "truncation": lambda a: (_u32(a) >> 16).astype(np.uint16),
    "ties toward odd": lambda a: ((_u32(a) + 0x7FFF + (1 - ((_u32(a) >> 16) & 1))) >> 16).astype(np.uint16),
    "ties down (lsb term dropped)": lambda a: ((_u32(a) + 0x7FFF) >> 16).astype(np.uint16),
    "rounded from float64 directly": lambda a: np.array(
        [_direct_f64(float(v)) for v in np.asarray(a, np.float64).ravel()], np.uint16),
}


def _direct_f64(v: float) -> int:
    """Nearest bf16 of the float64 value itself (no float32 step), ties to even."""
    f = np.float32(v)
    b0 = int(np.array([f]).view(np.uint32)[0] >> 16)
    best = None
    for c in (b0 - 1, b0, b0 + 1):
        if not 0 <= c <= 0xFFFF or (c & 0x7F80) == 0x7F80:
            continue
        d = abs(float(_bits_to_f64(c)) - v)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mutations_are_caught(name):
    assert not _pins_hold(MUTANTS[name]), name
