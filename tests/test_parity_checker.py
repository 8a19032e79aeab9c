"""The parity checker must trip on a perturbation just beyond its bar (a control in the
sense of the prefill page, PR #196: perturb the OUTPUT, not a shared input)."""
import numpy as np

import parity


def test_f32_checker_passes_identity_and_trips_beyond_bar():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((32, 64)) * 5
    ok, _ = parity.check_f32(ref.astype(np.float32), ref)
    assert ok
    bad = ref.copy(); bad[3, 7] += 0.021
    assert not parity.check_f32(bad, ref)[0]
    bad = ref * (1 + 2e-3)
    assert not parity.check_f32(bad, ref)[0]
    bad = ref.copy(); bad[0, 0] = np.nan
    assert not parity.check_f32(bad, ref)[0]


def _bf16(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_checker_one_ulp_passes_and_beyond_the_bar_trips():
    rng = np.random.default_rng(1)
    vals = rng.standard_normal(4096) * 3
    ref = _bf16(vals)
    assert parity.check_bf16(ref, ref)[0]
    big = int(np.argmax(np.abs(vals)))                   # |v| > 4: one ulp is 2^-5 or more
    assert abs(vals[big]) > 4
    one = ref.copy(); one[big] = one[big] + 1
    assert parity.check_bf16(one, ref)[0]                # a rounding-boundary neighbour
    two = ref.copy(); two[big] = two[big] + 2
    assert not parity.check_bf16(two, ref)[0]            # two ulps = 0.0625 > 2e-2
    small = int(np.argmin(np.abs(vals - 0.3)))
    off = ref.copy()
    while parity.bf16_to_f64(off[small]) - parity.bf16_to_f64(ref[small]) <= 0.02:
        off[small] += 1                                  # the first bf16 value beyond +2e-2
    assert not parity.check_bf16(off, ref)[0]            # just over 2e-2 absolute, many ulps near 0.3
    near = ref.copy(); near[small] = _bf16([float(parity.bf16_to_f64(ref[small])) + 0.015])[0]
    assert parity.check_bf16(near, ref)[0]               # within 2e-2 absolute
    scaled = _bf16(vals * (1 + 2e-3))
    assert not parity.check_bf16(scaled, ref)[0]         # rel-L2 2e-3
    nan = ref.copy(); nan[0] = 0x7FC0
    assert not parity.check_bf16(nan, ref)[0]
    # across zero: +0 vs -0 is 0 ulps; smallest positive vs smallest negative is 2
    assert parity.bf16_ordinal(np.array([0x0000]))[0] == parity.bf16_ordinal(np.array([0x8000]))[0]
    assert parity.bf16_ordinal(np.array([0x0001]))[0] - parity.bf16_ordinal(np.array([0x8001]))[0] == 2


def test_exact_checker_trips_on_one_unit():
    a = np.arange(100, dtype=np.int32)
    b = a.copy(); b[50] += 1
    assert parity.check_exact(a, a)[0]
    assert not parity.check_exact(a, b)[0]
