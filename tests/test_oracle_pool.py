"""oracle.pool schedules oracle.moe over worker processes; its outputs must be moe_forward's."""
import numpy as np
import pytest

import moe_inputs
from oracle import moe, pool

MID = moe_inputs.MoEShape(num_experts=16, top_k=4, hidden=256, inter=128, n_tokens=40)


def test_pool_equals_moe_forward_on_layers_sharing_weights():
    layers = moe_inputs.make_inputs_multi(MID, [1, 7, 40], seed=13)
    zipf = moe_inputs.make_inputs_multi(moe_inputs.MoEShape(16, 4, 256, 128, 30, routing="zipf"), [30], seed=13)[30]
    named = {"n1": layers[1], "n7": layers[7], "n40": layers[40], "zipf": zipf}
    res = pool.layer_outputs(named, workers=3)
    for name, inp in named.items():
        ref = moe.moe_forward(inp)
        assert np.allclose(res[name]["out_f64"], ref["out_f64"], rtol=1e-12, atol=1e-15), name
        assert np.array_equal(res[name]["topk_idx"], ref["topk_idx"])


def test_pool_refuses_layers_with_different_weights():
    a = moe_inputs.make_inputs(MID, seed=1)
    b = moe_inputs.make_inputs(MID, seed=2)
    with pytest.raises(ValueError):
        pool.layer_outputs({"a": a, "b": b}, workers=1)


def test_pool_expert_subset_returns_only_those_pairs():
    inp = moe_inputs.make_inputs(MID, seed=14)
    res = pool.layer_outputs({"x": inp}, workers=2, experts=[0, 3])
    ref = moe.moe_forward(inp)
    idx = ref["topk_idx"].reshape(-1)
    want = {p for p in range(idx.size) if idx[p] in (0, 3)}
    assert set(res["x"]["y"]) == want and "out_f64" not in res["x"]
    for p in want:
        assert np.allclose(res["x"]["y"][p], ref["y"][p], rtol=1e-12, atol=1e-15)


def test_timing_split_is_reported_when_asked():
    inp = moe_inputs.make_workload("tiny", seed=0)
    timing = {}
    res = pool.layer_outputs({"t": inp}, 2, timing=timing)
    assert set(timing) == {"decode_s", "pairs_s"}
    assert timing["decode_s"] > 0.0 and timing["pairs_s"] > 0.0
    # the same outputs with or without the timing dict
    again = pool.layer_outputs({"t": inp}, 2)
    assert np.array_equal(res["t"]["out_f64"], again["t"]["out_f64"])
