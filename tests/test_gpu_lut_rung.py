"""The LUT rung on the GPU (plan.rung = QTIP_RUNG_LUT) against the oracle (oracle.lut_rung).

Integer-exact work is compared bit for bit: qtip_expert_matmul through an integer codebook with
scale 1 and one-hot activation rows returns the decoded weights exactly, and qtip_moe_dequantize
returns bf16(codebook[state]) for every weight.  Layers meet the parity bar (max-abs 2e-2 and
rel-L2 1e-3; bf16 outputs within 2e-2 or one bf16 ulp per element): the tiny layer with every arm
and both output types, mid-size layers with ragged tiles on both arms, every kernel configuration
and both activation layouts, and every token of every V4-shaped LUT-rung workload in the plan the
benchmark times."""
import os
import subprocess
import sys

import numpy as np
import pytest

import moe_inputs
import parity
import trellis_quantized_moe_expert_amd as q
from gpu_util import Layer, say
from moe_inputs.device import weights_to_device
from oracle import lut_rung, moe, numerics, pool

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import oracle_v4_job  # noqa: E402

MID = moe_inputs.MoEShape(num_experts=16, top_k=4, hidden=512, inter=256, n_tokens=100, rung="lut")


def check(got, ref, out_dtype):
    if out_dtype == "f32":
        ok, st = parity.check_f32(got, ref["out_f64"])
    else:
        ok, st = parity.check_bf16(got, ref["out"])
    assert ok, st
    return st


def int_codebook():
    s = np.arange(512)
    return np.stack([s % 13 - 6, 7 - s % 11], axis=1).astype(np.float16)


@pytest.mark.parametrize("arm", [q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED])
@pytest.mark.parametrize("rows,cols", [(64, 128), (32, 384), (32, 512), (48, 640), (2048, 4096), (4096, 2048)])
def test_matmul_decodes_an_integer_codebook_exactly(arm, rows, cols):
    """y = a W^T with one-hot rows of a picks columns of W; with integer weights, scale 1 and
    exact fp32 sums the GPU must return the decoded weights bit for bit (the wrap region of each
    row included: the columns near cols-1)."""
    import torch
    rng = np.random.default_rng(rows + cols + arm)
    E = 2
    codes = rng.integers(0, 256, size=(E, rows, cols // 4), dtype=np.uint8)
    scales = np.ones((E, rows), np.float16)
    cb = int_codebook()
    picks = [0, 1, 2, 3, 31, 32, 127, cols - 9, cols - 8, cols - 3, cols - 2, cols - 1]
    a = np.zeros((len(picks), cols), np.float32)
    a[np.arange(len(picks)), picks] = 1.0
    a_bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
    plan = q.qtip_moe_plan(q.make_desc(E, 1, 128, 128, 1, rung=q.QTIP_RUNG_LUT), 0)
    say(f"LUT-rung matmul arm={arm} rows={rows} cols={cols}")
    for e in range(E):
        y = torch.full((len(picks), rows), np.nan, dtype=torch.float32, device="cuda:0")
        units = np.array([[e, 0, len(picks)]], np.int32)
        q.qtip_expert_matmul(plan, arm, dev(codes), dev(scales.view(np.int16)), dev(cb.view(np.int16)), E, rows, cols,
                             dev(a_bits.view(np.int16)), len(picks), dev(units), 1, y)
        torch.cuda.synchronize()
        w = lut_rung.decode_declared(lut_rung.stored_rows(codes[e]), cb)
        assert np.array_equal(y.cpu().numpy(), w[:, picks].T.astype(np.float32)), e
    q.qtip_moe_plan_destroy(plan)


@pytest.mark.parametrize("name,shape,experts", [("tiny", moe_inputs.WORKLOADS["lut_tiny"], [0, 7]),
                                                ("mid", MID, [0, 15]),
                                                ("v4", moe_inputs.WORKLOADS["lut_v4_decode_n32"], [0, 255])])
def test_dequantize_is_bit_exact(name, shape, experts):
    import torch
    inp = moe_inputs.make_inputs(shape, seed=2, n_tokens=4)
    layer = Layer(inp, max_tokens=4)
    s = inp.shape
    for e in experts:
        for m, codes in enumerate((inp.codes_gate, inp.codes_up, inp.codes_down)):
            rows, cols = (s.hidden, s.inter) if m == 2 else (s.inter, s.hidden)
            out = torch.empty((rows, cols), dtype=torch.int16, device="cuda:0")
            q.qtip_moe_dequantize(layer.plan, layer.w, m, e, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy().view(np.uint16)
            want = numerics.f64_to_bf16_bits(lut_rung.decode_declared(lut_rung.stored_rows(codes[e]), inp.lut))
            assert np.array_equal(got, want), (name, e, m)
    layer.close()


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("arm", [q.QTIP_ARM_AUTO, q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED, q.QTIP_ARM_DEQUANT])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_tiny_lut_layer_full_parity(seed, arm, out_dtype):
    inp = moe_inputs.make_workload("lut_tiny", seed=seed)
    say(f"LUT-rung forward tiny seed={seed} arm={arm} out={out_dtype}")
    layer = Layer(inp, arm=arm, out_dtype=out_dtype)
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    assert st["last_arm"] == q.qtip_moe_select_arm(layer.plan, 16)
    layer.close()
    check(got, moe.moe_forward(inp, out_dtype=out_dtype), out_dtype)


# an odd number of 128-input blocks in both passes (3 in gate+up, 5 in down): the grouped arm walks
# the blocks of a row in descending order over two alternating buffers, so odd counts end on the
# other buffer
ODD = moe_inputs.MoEShape(num_experts=12, top_k=3, hidden=384, inter=640, n_tokens=60, rung="lut")


@pytest.mark.parametrize("arm", [q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED])
@pytest.mark.parametrize("n", [1, 7, 60, 90])
def test_lut_layer_with_odd_block_counts(arm, n):
    inp = moe_inputs.make_inputs(ODD, seed=5, n_tokens=n)
    say(f"LUT-rung forward odd blocks n={n} arm={arm}")
    layer = Layer(inp, arm=arm, out_dtype="f32", max_tokens=90)
    got = layer.forward(inp)
    layer.close()
    check(got, moe.moe_forward(inp), "f32")


@pytest.mark.parametrize("arm", [q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED])
@pytest.mark.parametrize("n", [1, 9, 100, 300])
def test_mid_lut_layer_ragged_tiles(arm, n):
    inp = moe_inputs.make_inputs(MID, seed=3, n_tokens=n)
    say(f"LUT-rung forward mid n={n} arm={arm}")
    layer = Layer(inp, arm=arm, out_dtype="f32", max_tokens=300)
    got = layer.forward(inp)
    layer.close()
    check(got, moe.moe_forward(inp), "f32")


def test_lut_decode_floor_switches_arms_at_five_tokens():
    """The plan's default decode floor on this rung (4, a token count whatever the shape): 4 tokens
    take the GEMV arm, 5 the grouped arm; both match the oracle token by token."""
    inps = moe_inputs.make_inputs_multi(MID, [4, 5], seed=22)
    layer = Layer(inps[4], out_dtype="f32", max_tokens=5)
    for n, arm in ((4, q.QTIP_ARM_GEMV), (5, q.QTIP_ARM_GROUPED)):
        say(f"LUT-rung forward V4 floor n={n}")
        got = layer.forward(inps[n])
        assert q.qtip_moe_stats(layer.plan)["last_arm"] == arm
        check(got, moe.moe_forward(inps[n]), "f32")
    layer.close()


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11])
@pytest.mark.parametrize("arm", [q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED])
def test_lut_kernel_variants(variant, arm):
    inp = moe_inputs.make_inputs(MID, seed=8, n_tokens=260)
    say(f"LUT-rung forward variant={variant} arm={arm}")
    s = inp.shape
    layer = Layer(inp, arm=arm)
    q.qtip_moe_plan_destroy(layer.plan)
    layer.plan = q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, 260, arm, variant,
                                             q.QTIP_OUT_F32, 0, rung=q.QTIP_RUNG_LUT), 0)
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    key = "grouped_variant_launches" if arm == q.QTIP_ARM_GROUPED else "gemv_variant_launches"
    ran = {v for v, c in enumerate(st[key]) if c}
    sched = q.qtip_moe_plan_schedule(layer.plan, 260)
    assert ran == {sched["gate_up"]["variant"], sched["down"]["variant"]}
    layer.close()
    ref = moe.moe_forward(inp)
    assert ref["bins"]["counts"].max() > 64
    check(got, ref, "f32")


@pytest.mark.parametrize("layout", [q.QTIP_ACT_ROWS, q.QTIP_ACT_FRAGMENTS])
@pytest.mark.parametrize("n", [1, 17, 260])
def test_lut_activation_layouts(layout, n):
    import torch
    inp = moe_inputs.make_inputs(MID, seed=9, n_tokens=n)
    say(f"LUT-rung forward layout={layout} n={n}")
    s = inp.shape
    layer = Layer(inp, arm=q.QTIP_ARM_GROUPED, max_tokens=260)
    q.qtip_moe_plan_destroy(layer.plan)
    layer.plan = q.qtip_moe_plan(q.make_desc(s.num_experts, s.top_k, s.hidden, s.inter, 260, q.QTIP_ARM_GROUPED, 0,
                                             q.QTIP_OUT_F32, 0, act_layout=layout, rung=q.QTIP_RUNG_LUT), 0)
    layer.ws = torch.empty(q.qtip_moe_plan_info(layer.plan)["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
    got = layer.forward(inp)
    layer.close()
    check(got, moe.moe_forward(inp), "f32")


NAMES = oracle_v4_job.LUT_UNIFORM + oracle_v4_job.LUT_SKEWED


@pytest.fixture(scope="module")
def lut_oracle(tmp_path_factory):
    path = tmp_path_factory.mktemp("oracle_lut") / "lut.npz"
    cmd = [sys.executable, "-u", os.path.join(HERE, "oracle_v4_job.py"), "--out", str(path), "--rung", "lut",
           "--workers", str(pool.default_workers())]
    say("starting the LUT-rung V4 oracle job: " + " ".join(cmd[2:]))
    res = subprocess.run(cmd, timeout=1500, capture_output=True, text=True)
    say(res.stdout[-1500:] + res.stderr[-1500:])
    assert res.returncode == 0
    with np.load(path) as z:
        return {name: z[name] for name in NAMES}


@pytest.fixture(scope="module")
def lut_inputs():
    layers = oracle_v4_job.v4_layers("lut")
    return layers, weights_to_device(layers[NAMES[0]])


@pytest.mark.timeout(1800)
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", NAMES)
def test_v4_lut_every_token_matches_the_oracle(name, out_dtype, lut_inputs, lut_oracle):
    layers, dw = lut_inputs
    inp = layers[name]
    n = inp.shape.n_tokens
    say(f"LUT-rung V4 full parity {name} n={n} out={out_dtype}")
    layer = Layer(inp, out_dtype=out_dtype, weights=dw)
    got = layer.forward(inp)
    st = q.qtip_moe_stats(layer.plan)
    layer.close()
    assert st["last_arm"] == q.QTIP_ARM_GROUPED
    ref = lut_oracle[name]
    if out_dtype == "f32":
        ok, stats = parity.check_f32(got, ref)
    else:
        ok, stats = parity.check_bf16(got, numerics.f64_to_bf16_bits(ref))
    say(f"  {stats}")
    assert ok, stats
