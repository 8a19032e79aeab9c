"""bf16 rounding used at the path's declared rounding points (oracle side).

bf16 keeps the top 16 bits of an IEEE float32.  Rounding a float32 value to bf16
to nearest, ties to even, adds 0x7FFF plus the lowest kept bit to the 32-bit
pattern and truncates; every value handled here is finite.
"""
import numpy as np


def bf16_round(a) -> np.ndarray:
    """float64/float32 -> nearest bf16 value (ties to even), returned as float64.

    The input is first rounded to float32 (the path holds these values in fp32
    before narrowing them), then to bf16.
    """
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(a) -> np.ndarray:
    """float64 -> bf16 bit patterns (round to float32, then to bf16, nearest-even)."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
