"""Top-k routing and expert binning, oracle side (test infrastructure only).

Sources:
* Binning and the m-tile walk: the gate-the-grouped-GEMM page (PR #167 "gate the
  trellis grouped GEMM on m-tile occupancy, not token count"), section "The cause
  is a threshold, not a kernel defect": (token, expert) pairs are sorted by expert
  and the kernel walks sum_e ceil(count_e / GROUPED_TILE_M) m-tiles.
* Router weights: the workload definition gives softmax over the top-k logits; the
  pages are silent on the formula, so the plain reading is used (no extra scale, no
  shared expert).

Readings where the pages are silent:
* top-k picks the k largest logits in descending order; equal logits go to the
  lower expert index.
* pair id p = t*k + j for the j-th choice of token t; within an expert's bin
  pairs keep ascending pair id (a stable sort), which makes the binning unique.
* tiles are listed expert by expert in ascending expert order, each expert's bin
  cut into consecutive tiles of tile_m pairs, the last one partial.
"""
from __future__ import annotations

import math

import numpy as np


def route_topk_bruteforce(logits: np.ndarray, k: int):
    """Per token: sort experts by (-logit, index) with Python's sorted; softmax in float64."""
    n, E = logits.shape
    idx = np.zeros((n, k), np.int32)
    w = np.zeros((n, k), np.float32)
    for t in range(n):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        idx[t] = order
        sel = [row[e] for e in order]
        m = max(sel)
        ex = [math.exp(v - m) for v in sel]
        z = sum(ex)
        w[t] = [v / z for v in ex]
    return idx, w


def route_topk(logits: np.ndarray, k: int):
    """Vectorised top-k: a stable argsort of the negated logits keeps ties in index order."""
    logits = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return order, w


def bin_pairs(topk_idx: np.ndarray, num_experts: int, tile_m: int) -> dict:
    """Counting sort of pairs by expert (stable in pair id) and the m-tile map."""
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int32)
    tiles = []
    for e in range(num_experts):
        start = int(offsets[e])
        for q in range(0, int(counts[e]), tile_m):
            tiles.append((e, start + q, min(tile_m, int(counts[e]) - q)))
    tile_map = np.array(tiles, np.int32).reshape(-1, 3)
    return {"counts": counts, "offsets": offsets, "sorted_pair": sorted_pair,
            "tile_map": tile_map, "n_tiles": len(tiles)}


def bin_pairs_bruteforce(topk_idx: np.ndarray, num_experts: int, tile_m: int) -> dict:
    """The same result by explicit Python loops (sorted by (expert, pair id))."""
    n, k = topk_idx.shape
    pairs = [(int(topk_idx[t][j]), t * k + j) for t in range(n) for j in range(k)]
    pairs.sort()
    counts = [0] * num_experts
    for e, _ in pairs:
        counts[e] += 1
    offsets = [0]
    for e in range(num_experts):
        offsets.append(offsets[-1] + counts[e])
    tiles = []
    for e in range(num_experts):
        c = counts[e]
        q = 0
        while q < c:
            tiles.append((e, offsets[e] + q, min(tile_m, c - q)))
            q += tile_m
    return {"counts": np.array(counts, np.int32), "offsets": np.array(offsets, np.int32),
            "sorted_pair": np.array([p for _, p in pairs], np.int32),
            "tile_map": np.array(tiles, np.int32).reshape(-1, 3), "n_tiles": len(tiles)}
