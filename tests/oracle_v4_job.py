"""Declared-mode oracle outputs of every V4-shaped workload, saved to an .npz file.

All V4 workloads draw the same seed-0 expert weights, so the oracle decodes each expert once for
all of them (oracle.pool).  Run as its own process (the full-size parity tests start it with
subprocess), so that its worker pool forks from a process that has not touched a GPU:

    python tests/oracle_v4_job.py --out PATH [--workers N] [--rung bitshift|lut]
"""
import argparse
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import moe_inputs  # noqa: E402
from oracle import pool  # noqa: E402

UNIFORM = ["v4_decode_n32", "v4_mid_n128", "v4_mid_n512", "v4_full_n683", "v4_full_n1024"]
SKEWED = ["v4_zipf_n256"]
# the same layers with LUT-rung experts
LUT_UNIFORM = ["lut_v4_decode_n32", "lut_v4_mid_n128", "lut_v4_mid_n512", "lut_v4_full_n1024"]
LUT_SKEWED = ["lut_v4_zipf_n256"]
RUNGS = {"bitshift": (UNIFORM, SKEWED), "lut": (LUT_UNIFORM, LUT_SKEWED)}


def v4_layers(rung: str = "bitshift") -> dict:
    """Every V4 workload of the rung, the uniform ones sharing one weight draw
    (moe_inputs.make_inputs_multi)."""
    uniform, skewed = RUNGS[rung]
    W = moe_inputs.WORKLOADS
    uni = moe_inputs.make_inputs_multi(W[uniform[0]], [W[n].n_tokens for n in uniform], seed=0)
    layers = {name: uni[W[name].n_tokens] for name in uniform}
    for name in skewed:
        layers[name] = moe_inputs.make_inputs_multi(W[name], [W[name].n_tokens], seed=0)[W[name].n_tokens]
    return layers


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--workers", type=int, default=pool.default_workers())
    ap.add_argument("--rung", choices=sorted(RUNGS), default="bitshift")
    args = ap.parse_args()
    t0 = time.perf_counter()
    say = lambda *a: print(*a, flush=True)
    layers = v4_layers(args.rung)
    say(f"oracle job: {len(layers)} V4 layers drawn in {time.perf_counter() - t0:.1f} s; {args.workers} workers")
    res = pool.layer_outputs(layers, args.workers, log=say)
    np.savez(args.out, **{name: res[name]["out_f64"] for name in layers})
    say(f"oracle job: done in {time.perf_counter() - t0:.1f} s")


if __name__ == "__main__":
    main()
