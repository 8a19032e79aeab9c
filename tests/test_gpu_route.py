"""GPU routing and binning vs the oracle: indices, counts, offsets, sorted pairs and the tile
map must match bit for bit (routing is integer work decided by float compares)."""
import numpy as np
import pytest

import moe_inputs
import trellis_quantized_moe_expert_amd as q
from gpu_util import say
from oracle import routing

pytestmark = pytest.mark.gpu


def run_route(logits, E, k, tile_m=0):
    import torch
    n = logits.shape[0]
    plan = q.qtip_moe_plan(q.make_desc(E, k, 128, 128, n, tile_m=tile_m), 0)
    tm = q.qtip_moe_plan_info(plan)["tile_m"]
    dev = lambda *shape, dt=torch.int32: torch.full(shape, -7, dtype=dt, device="cuda:0")
    lg = torch.from_numpy(np.ascontiguousarray(logits)).to("cuda:0")
    out = dict(topk_idx=dev(n, k), topk_w=dev(n, k, dt=torch.float32), counts=dev(E), offsets=dev(E + 1),
               sorted_pair=dev(n * k), tile_map=dev(n * k, 3), n_tiles=dev(1))
    q.qtip_moe_route(plan, lg, n, out["topk_idx"], out["topk_w"], out["counts"], out["offsets"], out["sorted_pair"],
                     out["tile_map"], out["n_tiles"])
    torch.cuda.synchronize()
    q.qtip_moe_plan_destroy(plan)
    res = {kk: v.cpu().numpy() for kk, v in out.items()}
    res["n_tiles"] = int(res["n_tiles"][0])
    res["tile_map"] = res["tile_map"][:res["n_tiles"]]
    return res, tm


def compare(logits, E, k, tile_m=0):
    g, tm = run_route(logits, E, k, tile_m)
    idx, w = routing.route_topk(logits, k)
    b = routing.bin_pairs(idx, E, tm)
    assert np.array_equal(g["topk_idx"], idx)
    assert np.allclose(g["topk_w"], w, rtol=2e-6, atol=1e-7)
    for key in ("counts", "offsets", "sorted_pair", "tile_map"):
        assert np.array_equal(g[key], b[key]), key
    assert g["n_tiles"] == b["n_tiles"]


@pytest.mark.parametrize("name", list(moe_inputs.WORKLOADS))
def test_route_bitexact_workload_logits(name):
    s = moe_inputs.WORKLOADS[name]
    say(f"route {name}: n={s.n_tokens} E={s.num_experts} k={s.top_k} routing={s.routing}")
    compare(moe_inputs.draw_logits(s, seed=0), s.num_experts, s.top_k)


@pytest.mark.parametrize("tile_m", [16, 32, 64])
def test_route_bitexact_ties_and_tile_heights(tile_m):
    rng = np.random.default_rng(tile_m)
    logits = np.round(rng.standard_normal((300, 64)) * 1.5).astype(np.float32)   # heavy ties
    logits[0] = 0.0
    logits[1] = -0.0
    logits[2, ::2] = -0.0
    say(f"route ties tile_m={tile_m}")
    compare(logits, 64, 5, tile_m)


@pytest.mark.parametrize("n,E,k", [(1, 8, 2), (3, 1024, 32), (2000, 256, 8), (700, 1, 1), (5, 6, 6)])
def test_route_bitexact_edge_shapes(n, E, k):
    rng = np.random.default_rng(n + E)
    say(f"route edge n={n} E={E} k={k}")
    compare(rng.standard_normal((n, E)).astype(np.float32), E, k)


@pytest.mark.parametrize("n,E,k", [(16, 256, 6), (17, 256, 6), (16, 256, 20), (15, 200, 32), (16, 1, 1),
                                   (14, 17, 16), (16, 1024, 8), (17, 1024, 8), (16, 300, 4), (12, 512, 3)])
def test_route_bitexact_small_batches_with_ties(n, E, k):
    # batches of up to 16 tokens are routed and binned by one workgroup (a token per wave),
    # larger ones by the two launches; the shapes straddle that limit and each logits-per-lane
    # instantiation (E up to 256, 512, 1024)
    rng = np.random.default_rng(7 * n + E)
    logits = np.round(rng.standard_normal((n, E)) * 1.5).astype(np.float32)   # heavy ties
    logits[0] = 0.0
    logits[-1, ::3] = -0.0
    say(f"route small batch n={n} E={E} k={k}")
    compare(logits, E, k)


def test_route_skewed_hot_expert():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((1500, 32)).astype(np.float32)
    logits[:, 3] += 10.0          # every token picks expert 3: one bin of 1500 pairs
    say("route hot expert")
    compare(logits, 32, 4)


def test_lut_gather_calibration_runs():
    import torch
    n = torch.cuda.get_device_properties(0).multi_processor_count * 1024
    sink = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    rate = q.qtip_measure_lut_gather(200, sink, n)
    say(f"LDS random gather: {rate / 1e12:.2f} T lookups/s")
    assert 1e12 < rate < 2e13
    with pytest.raises(q.QtipError):
        q.qtip_measure_lut_gather(10, sink, 16)          # sink too small: refused, nothing launched
