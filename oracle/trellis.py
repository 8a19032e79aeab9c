"""Bitshift-trellis decode, oracle side (test infrastructure only).

What is decoded (source: the arch-specialise page, PR #99 "arch-specialise the
trellis grouped GEMM", section "The two levers" item 2 "Contiguous-run decode":
packed 2-bit bytes cross memory, each weight's state is a window of the bit
stream, and a run of consecutive symbols of one weight row can be seeded once
from its window and then stepped by the trellis recurrence).  The pages do not
fix the bit layout; the reading used here (stated once, also documented with the
C ABI) is:

* A matrix with `rows` output rows and `cols` inputs stores each row as an
  independent stream of `cols` 2-bit symbols in `cols/4` bytes.  Symbol c of a
  row is bits [2(c mod 4), 2(c mod 4)+2) of byte c//4 (little-endian, LSB first).
* The state of weight (r, c) is the 16-bit window of 8 symbols starting at c,
  read circularly within the row (tail-biting, so exactly 2 bits per weight are
  stored):  state(r, c) = sum_{j=0..7} sym(r, (c + j) mod cols) * 4**j.
  Equivalently, stepping one symbol: state(c+1) = (state(c) >> 2) | (sym(c+8) << 14).
* The weight value is LUT[state] (a 65536-entry fp16 table) times a per-row
  fp16 scale.  In the path's declared rounding the LUT value is narrowed to bf16
  and the scale multiplies the fp32 dot product afterwards.
* Storage (a layout, not part of the arithmetic; the pages give only "packed
  2-bit bytes"): a matrix's rows x cols/4 bytes are stored block-interleaved, the
  32 bytes of 16 consecutive rows for 128 consecutive inputs together (byte
  32k + c of row r at ((r // 16) * (cols // 128) + k) * 512 + (r % 16) * 32 + c).
  stored_rows() turns stored bytes back into rows; every decode below takes rows.
"""
from __future__ import annotations

import numpy as np

WINDOW_SYMBOLS = 8          # 16-bit state = 8 symbols of 2 bits
STATE_MASK = 0xFFFF


# ---------------------------------------------------------------------------------
# Brute force: bit by bit, pure Python.  For hand-built streams and tiny matrices.
# ---------------------------------------------------------------------------------
def symbols_bruteforce(row_bytes) -> list:
    """Symbols of one row, read bit by bit: symbol = bit(2q) + 2*bit(2q+1) of each byte."""
    out = []
    for b in row_bytes:
        b = int(b)
        for q in range(4):
            lo = (b >> (2 * q)) & 1
            hi = (b >> (2 * q + 1)) & 1
            out.append(lo + 2 * hi)
    return out


def window_state_bruteforce(syms, c: int) -> int:
    """The 16-bit state of position c: 8 symbols from c onward, circular, base 4, LSB first."""
    cols = len(syms)
    s = 0
    for j in range(WINDOW_SYMBOLS):
        s += syms[(c + j) % cols] * (4 ** j)
    return s


def run_states(syms, c0: int, length: int) -> list:
    """Contiguous-run decode: seed the state of c0 from its window once, then step.

    Each step drops the oldest symbol (shift right by 2) and brings in the symbol 8
    positions ahead at the top (bits 14-15), circularly within the row.
    """
    cols = len(syms)
    state = window_state_bruteforce(syms, c0)
    out = [state]
    for i in range(1, length):
        c = c0 + i
        incoming = syms[(c + WINDOW_SYMBOLS - 1) % cols]
        state = (state >> 2) | (incoming << 14)
        out.append(state)
    return out


def dense_weights_bruteforce(codes_2d, lut_f16, scales_f16=None, declared=True) -> np.ndarray:
    """Materialise one matrix's weights element by element (pure Python loops).

    declared=True: bf16(LUT[state]) without the scale (the scale is applied after the
    dot product); declared=False: float32(LUT[state]) * float32(scale[r]).
    """
    from .numerics import bf16_round
    rows = codes_2d.shape[0]
    lutv = np.asarray(lut_f16, dtype=np.float16).astype(np.float64)
    out = None
    for r in range(rows):
        syms = symbols_bruteforce(codes_2d[r])
        if out is None:
            out = np.zeros((rows, len(syms)), np.float64)
        for c in range(len(syms)):
            v = lutv[window_state_bruteforce(syms, c)]
            if declared:
                out[r, c] = float(bf16_round(v))
            else:
                out[r, c] = float(np.float32(v)) * float(np.float32(scales_f16[r]))
    return out


# ---------------------------------------------------------------------------------
# Vectorised numpy version of the same definition, for realistic sizes.
# ---------------------------------------------------------------------------------
def unpack_symbols(codes: np.ndarray) -> np.ndarray:
    """codes [..., cols/4] uint8 -> symbols [..., cols] uint8 (LSB-first within each byte)."""
    c = np.asarray(codes, dtype=np.uint8)
    parts = [(c >> (2 * q)) & 3 for q in range(4)]
    return np.stack(parts, axis=-1).reshape(*c.shape[:-1], c.shape[-1] * 4)


def window_states(codes: np.ndarray) -> np.ndarray:
    """codes [..., cols/4] -> states [..., cols] (int64), straight from the window definition."""
    syms = unpack_symbols(codes).astype(np.int64)
    state = np.zeros_like(syms)
    for j in range(WINDOW_SYMBOLS):
        state += np.roll(syms, -j, axis=-1) << (2 * j)
    return state


def stored_rows(stored: np.ndarray) -> np.ndarray:
    """The rows [..., rows, cols/4] of matrices held in the block-interleaved storage (the same
    number of bytes, in the same array shape): blocks [rows/16][cols/128][16 rows][32 bytes], i.e.
    byte 32k + c of row r sits at ((r // 16) * (cols // 128) + k) * 512 + (r % 16) * 32 + c.
    The layout needs whole blocks; smaller test matrices whose sides are not multiples of 16 rows
    and 128 inputs (shapes the library does not accept) are taken as stored row by row."""
    s = np.asarray(stored, np.uint8)
    *lead, rows, nb = s.shape
    if rows % 16 or nb % 32:
        return s
    b = s.reshape(*lead, rows // 16, nb // 32, 16, 32)
    return np.ascontiguousarray(np.swapaxes(b, -3, -2)).reshape(*lead, rows, nb)


def lut_bf16(lut_f16: np.ndarray) -> np.ndarray:
    """The LUT narrowed to bf16 (fp16 -> exact fp32 -> bf16 nearest-even), as float64."""
    from .numerics import bf16_round
    return bf16_round(np.asarray(lut_f16, dtype=np.float16).astype(np.float32))


def decode_declared(codes: np.ndarray, lut_f16: np.ndarray) -> np.ndarray:
    """Unscaled weights in the path's declared precision: bf16(LUT[state]) as float64."""
    return lut_bf16(lut_f16)[window_states(codes)]


def decode_exact(codes: np.ndarray, lut_f16: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """Scaled weights with no narrowing: float32(LUT[state]) * float32(scale[row]) as float64."""
    lutv = np.asarray(lut_f16, dtype=np.float16).astype(np.float64)
    w = lutv[window_states(codes)]
    return w * np.asarray(scales_f16, dtype=np.float16).astype(np.float64)[..., :, None]
