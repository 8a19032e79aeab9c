"""Every token of every V4-shaped workload against the declared-mode oracle, in the plan the
benchmark times (max_tokens = n, automatic arm and kernel configuration), with bf16 and fp32
outputs.

Workloads: E=256, top-6, hidden 4096, expert intermediate 2048, seed 0; n = 32, 128, 512, 683 and
1024 with uniform routing, and n = 256 with Zipf(1.1) expert popularity.  The oracle decodes each
expert once for all six layers (they share one weight draw) in a worker pool started as a separate
process (tests/oracle_v4_job.py).  Bars: fp32 outputs within max-abs 2e-2 and rel-L2 1e-3; bf16
outputs within rel-L2 1e-3 and, per element, within 2e-2 or one bf16 ulp of the oracle's own bf16
value.  The
launch counters must show the arm and kernel configurations the plan's schedule names."""
import os
import subprocess
import sys

import numpy as np
import pytest

import parity
import trellis_quantized_moe_expert_amd as q
from gpu_util import Layer, say
from moe_inputs.device import weights_to_device
from oracle import numerics, pool

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import oracle_v4_job  # noqa: E402

NAMES = oracle_v4_job.UNIFORM + oracle_v4_job.SKEWED


@pytest.fixture(scope="module")
def oracle_out(tmp_path_factory):
    path = tmp_path_factory.mktemp("oracle_v4") / "v4.npz"
    cmd = [sys.executable, "-u", os.path.join(HERE, "oracle_v4_job.py"), "--out", str(path),
           "--workers", str(pool.default_workers())]
    say("starting the V4 oracle job: " + " ".join(cmd[2:]))
    res = subprocess.run(cmd, timeout=1200, capture_output=True, text=True)
    say(res.stdout[-2000:] + res.stderr[-2000:])
    assert res.returncode == 0
    with np.load(path) as z:
        return {name: z[name] for name in NAMES}


@pytest.fixture(scope="module")
def v4_inputs():
    layers = oracle_v4_job.v4_layers()
    dw = weights_to_device(layers[NAMES[0]])
    return layers, dw


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", NAMES)
def test_every_token_matches_the_oracle(name, out_dtype, v4_inputs, oracle_out):
    layers, dw = v4_inputs
    inp = layers[name]
    n = inp.shape.n_tokens
    say(f"V4 full parity {name} n={n} out={out_dtype}")
    layer = Layer(inp, out_dtype=out_dtype, weights=dw)      # max_tokens = n, AUTO: the bench's plan
    sched = q.qtip_moe_plan_schedule(layer.plan, n)
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    assert st["last_arm"] == sched["arm"] == q.QTIP_ARM_GROUPED
    counts = st["grouped_variant_launches"]
    want = {sched["gate_up"]["variant"], sched["down"]["variant"]}
    assert sum(counts) == 2 and all(counts[v] >= 1 for v in want), (counts, sched)
    ref = oracle_out[name]
    if out_dtype == "f32":
        ok, stats = parity.check_f32(got, ref)
    else:
        ok, stats = parity.check_bf16(got, numerics.f64_to_bf16_bits(ref))
    say(f"  {stats}")
    assert ok, stats


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name", ["v4_decode_n32", "v4_mid_n128"])
def test_gemv_arm_every_token_matches_the_oracle(name, v4_inputs, oracle_out):
    """The same layers forced onto the GEMV arm: its default configurations there are 12-wave
    workgroups of 16-row tasks with up to three pairs per decode (n=32) and 8-wave workgroups of
    32-row tasks (n=128)."""
    layers, dw = v4_inputs
    inp = layers[name]
    n = inp.shape.n_tokens
    say(f"V4 full parity on the GEMV arm {name} n={n}")
    layer = Layer(inp, arm=q.QTIP_ARM_GEMV, weights=dw)
    sched = q.qtip_moe_plan_schedule(layer.plan, n)
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    assert st["last_arm"] == sched["arm"] == q.QTIP_ARM_GEMV
    assert sched["gate_up"]["variant"] == {"v4_decode_n32": 11, "v4_mid_n128": 4}[name]
    counts = st["gemv_variant_launches"]
    want = {sched["gate_up"]["variant"], sched["down"]["variant"]}
    assert sum(counts) == 2 and all(counts[v] >= 1 for v in want), (counts, sched)
    ok, stats = parity.check_f32(got, oracle_out[name])
    say(f"  {stats}")
    assert ok, stats
