"""Parity checks between the GPU path and the oracle.

Bars (floating point): with fp32 outputs, max-abs <= 2e-2 and rel-L2 <= 1e-3; with
bf16 outputs, rel-L2 <= 1e-3 and every element within 1 bf16 ulp of the oracle's
own bf16 value (both sides round once at the end; a value close to a rounding
boundary may land on either neighbour).  Integer work (routing, binning, decode
through an integer LUT) must match exactly.
"""
import numpy as np

F32_MAX_ABS = 2e-2
REL_L2 = 1e-3


def bf16_ordinal(bits):
    """Map bf16 bit patterns to integers whose difference counts ulps (sign-magnitude order)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    d = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / d) if d > 0 else float(np.linalg.norm(a - b))


def check_f32(gpu, ref_f64, max_abs=F32_MAX_ABS, rl2=REL_L2):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref_f64, np.float64)
    if gpu.shape != ref.shape or not np.all(np.isfinite(gpu)):
        return False, {"reason": "shape or non-finite"}
    ma = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    r = rel_l2(gpu, ref) if gpu.size else 0.0
    return (ma <= max_abs and r <= rl2), {"max_abs": ma, "rel_l2": r}


def check_bf16(gpu_bits, ref_bits, rl2=REL_L2):
    g = np.asarray(gpu_bits, np.uint16)
    r = np.asarray(ref_bits, np.uint16)
    if g.shape != r.shape:
        return False, {"reason": "shape"}
    gv = bf16_to_f64(g)
    if not np.all(np.isfinite(gv)):
        return False, {"reason": "non-finite"}
    ulps = int(np.max(np.abs(bf16_ordinal(g) - bf16_ordinal(r)))) if g.size else 0
    rr = rel_l2(gv, bf16_to_f64(r)) if g.size else 0.0
    return (ulps <= 1 and rr <= rl2), {"max_ulps": ulps, "rel_l2": rr}


def check_exact(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    ok = a.shape == b.shape and np.array_equal(a, b)
    return ok, {"mismatches": int(np.sum(a != b)) if a.shape == b.shape else -1}
