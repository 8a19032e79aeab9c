"""Parity checks between the GPU path and the oracle.

Bars (floating point), max-abs 2e-2 and rel-L2 1e-3 in both output types: with fp32
outputs, every element within 2e-2 of the oracle and rel-L2 <= 1e-3; with bf16 outputs,
every element within 2e-2 of the oracle's own bf16 value or one bf16 ulp from it, and
rel-L2 <= 1e-3 (both sides round once at the end; a value close to a rounding boundary
may land on either neighbour, and above 2 in magnitude one bf16 ulp exceeds 2e-2).  Integer work (routing, binning, decode
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
    if not gpu.size:
        return True, {"max_abs": 0.0, "rel_l2": 0.0}
    d = np.abs(gpu - ref)
    i = int(np.argmax(d))
    ma = float(d.flat[i])
    r = rel_l2(gpu, ref)
    return (ma <= max_abs and r <= rl2), {"max_abs": ma, "rel_l2": r, "worst": (float(gpu.flat[i]), float(ref.flat[i]))}


def check_bf16(gpu_bits, ref_bits, rl2=REL_L2, max_abs=F32_MAX_ABS):
    """Every element within max_abs of the oracle's bf16 value or one bf16 ulp from it (a value
    next to a rounding boundary may land on either neighbour, and above 2 in magnitude one bf16
    ulp exceeds 2e-2), and rel-L2 <= rl2 over the whole output."""
    g = np.asarray(gpu_bits, np.uint16)
    r = np.asarray(ref_bits, np.uint16)
    if g.shape != r.shape:
        return False, {"reason": "shape"}
    gv = bf16_to_f64(g)
    if not np.all(np.isfinite(gv)):
        return False, {"reason": "non-finite"}
    if not g.size:
        return True, {"max_ulps": 0, "max_abs": 0.0, "rel_l2": 0.0, "beyond": 0}
    rv = bf16_to_f64(r)
    ulps = np.abs(bf16_ordinal(g) - bf16_ordinal(r))
    d = np.abs(gv - rv)
    beyond = (ulps > 1) & (d > max_abs)
    rr = rel_l2(gv, rv)
    iu = int(np.argmax(ulps))
    ia = int(np.argmax(d))
    st = {"max_ulps": int(ulps.flat[iu]), "at_max_ulps": (float(gv.flat[iu]), float(rv.flat[iu])),
          "max_abs": float(d.flat[ia]), "at_max_abs": (float(gv.flat[ia]), float(rv.flat[ia])),
          "rel_l2": rr, "beyond": int(np.sum(beyond)), "off_by_one_ulp": int(np.sum(ulps == 1))}
    return (not beyond.any() and rr <= rl2), st


def check_exact(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    ok = a.shape == b.shape and np.array_equal(a, b)
    return ok, {"mismatches": int(np.sum(a != b)) if a.shape == b.shape else -1}
