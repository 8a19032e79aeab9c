"""The oracle layer over a process pool, for layers too large for one core (TEST INFRASTRUCTURE ONLY).

This module adds scheduling only: it routes and bins each layer with oracle.routing, decodes
each woken expert once with oracle.moe.decode_expert, evaluates that expert's binned pairs of
every layer with oracle.moe.expert_pairs, and combines with oracle.moe.combine.  All the
arithmetic is those functions'; the result equals oracle.moe.moe_forward on each layer.

Several layers may share one set of expert weights (the same draw of moe_inputs at different
batch sizes), so one decode of an expert serves all of them.  Workers are forked from the
calling process, so call it from a process that has not initialised a GPU (a subprocess of a GPU
test, or a benchmark before its first device call); each worker runs numpy with one BLAS thread.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

from . import moe, routing

_JOB = None  # (layers, bins) inherited by forked workers


def _init_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _expert_task(e: int):
    layers, bins = _JOB
    first = next(iter(layers.values()))
    weights = None
    out = {}
    t_decode = t_pairs = 0.0
    for name, inp in layers.items():
        b = bins[name]
        start, cnt = int(b["offsets"][e]), int(b["counts"][e])
        if cnt == 0:
            continue
        pids = b["sorted_pair"][start:start + cnt]
        if weights is None:
            t0 = time.perf_counter()
            weights = moe.decode_expert(first, e)
            t_decode += time.perf_counter() - t0
        t0 = time.perf_counter()
        ye, _ = moe.expert_pairs(inp, e, pids, weights=weights)
        t_pairs += time.perf_counter() - t0
        out[name] = (np.asarray(pids), ye)
    return e, out, (t_decode, t_pairs)


def same_weights(a, b) -> bool:
    return all(np.array_equal(getattr(a, f), getattr(b, f)) for f in
               ("lut", "codes_gate", "codes_up", "codes_down", "scale_gate", "scale_up", "scale_down"))


def layer_outputs(layers: dict, workers: int, experts=None, tile_m: int = 16, log=None, timing=None) -> dict:
    """Declared-mode outputs of several layers that share expert weights.

    layers: {name: MoEInputs}; every entry must hold the same weights.  experts: expert ids to
    evaluate (default: every expert some layer wakes); with a subset, only the pairs of those
    experts are computed and no combine is done.  Returns {name: {"out_f64", "topk_idx",
    "topk_w", "bins", "y"}} ("out_f64" only when every woken expert was evaluated).  If `timing`
    is a dict it receives the worker seconds spent decoding experts ("decode_s") and evaluating
    their pairs ("pairs_s", the matmuls), summed over workers."""
    global _JOB
    names = list(layers)
    first = layers[names[0]]
    for name in names[1:]:
        if not same_weights(first, layers[name]):
            raise ValueError(f"layer {name} does not share the weights of {names[0]}")
    E, k, H = first.shape.num_experts, first.shape.top_k, first.shape.hidden
    routed = {}
    bins = {}
    for name in names:
        idx, w = routing.route_topk(layers[name].logits, k)
        routed[name] = (idx, w)
        bins[name] = routing.bin_pairs(idx, E, tile_m)
    woken = sorted({e for name in names for e in np.nonzero(bins[name]["counts"])[0].tolist()})
    todo = woken if experts is None else [e for e in experts if e in set(woken)]
    _JOB = (layers, bins)
    y = {name: {} for name in names}
    t0 = time.perf_counter()
    ctx = mp.get_context("fork")
    workers = max(1, min(workers, len(todo)))
    with ctx.Pool(workers, initializer=_init_worker) as pool:
        t_decode = t_pairs = 0.0
        for i, (e, res, (td, tp)) in enumerate(pool.imap_unordered(_expert_task, todo, chunksize=1)):
            t_decode += td
            t_pairs += tp
            for name, (pids, ye) in res.items():
                for q, p in enumerate(pids):
                    y[name][int(p)] = ye[q]
            if log and (i + 1) % 32 == 0:
                log(f"oracle pool: {i + 1}/{len(todo)} experts in {time.perf_counter() - t0:.1f} s")
    _JOB = None
    if timing is not None:
        timing["decode_s"] = t_decode
        timing["pairs_s"] = t_pairs
    out = {}
    for name in names:
        idx, w = routed[name]
        r = {"topk_idx": idx, "topk_w": w, "bins": bins[name], "y": y[name]}
        if experts is None:
            n = layers[name].logits.shape[0]
            r["out_f64"] = moe.combine(y[name], w, list(range(n)), k, H)
        out[name] = r
    return out


def default_workers(cap: int = 16) -> int:
    """Host cores this process may use, at most `cap`."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(cap, n))
