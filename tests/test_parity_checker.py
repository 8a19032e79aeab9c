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


def test_bf16_checker_one_ulp_passes_two_ulps_trip():
    rng = np.random.default_rng(1)
    ref = (rng.standard_normal(4096).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert parity.check_bf16(ref, ref)[0]
    one = ref.copy(); one[5] = one[5] + 1
    assert parity.check_bf16(one, ref)[0]
    two = ref.copy(); two[5] = two[5] + 2
    assert not parity.check_bf16(two, ref)[0]
    # across zero: +0 vs -0 is 0 ulps; smallest positive vs smallest negative is 2
    assert parity.bf16_ordinal(np.array([0x0000]))[0] == parity.bf16_ordinal(np.array([0x8000]))[0]
    assert parity.bf16_ordinal(np.array([0x0001]))[0] - parity.bf16_ordinal(np.array([0x8001]))[0] == 2


def test_exact_checker_trips_on_one_unit():
    a = np.arange(100, dtype=np.int32)
    b = a.copy(); b[50] += 1
    assert parity.check_exact(a, a)[0]
    assert not parity.check_exact(a, b)[0]
