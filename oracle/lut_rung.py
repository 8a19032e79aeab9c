"""Decode of the LUT rung (the "qtip2" format), oracle side (test infrastructure only).

The pages name two 2-bit trellis rungs of the same MoE expert path: the bitshift rung ("qtip2b")
and the LUT rung ("qtip2"), whose grouped kernel (qtip_lut_grouped_gemm_kernel) is the one the
m-tile page measures (PR #167, "The regression"; "Applied to both rungs": the same dispatch gate
governs both), and whose own gate the prefill page leaves unmeasured (PR #196, "Follow-ups found,
not fixed here").  The pages never define the LUT rung's format.  The reading used here (stated
once, also documented with the C ABI):

* The packed stream is the bitshift rung's: a matrix row of `cols` weights is `cols` 2-bit
  symbols in cols/4 bytes, symbol c = bits [2(c mod 4), +2) of byte c//4, rows independent and
  read circularly (2 bits per weight stored).
* Weights are decoded in pairs (2i, 2i+1): one trellis step emits a 2-D vector.  The state of
  pair i is the Q-bit window of the row's bit stream starting at bit 4i, read circularly:
      state(r, i) = sum_{b<Q} bit(r, (4i + b) mod 2cols) * 2**b,
  i.e. the low Q bits of the bitshift rung's 16-bit state of weight 2i.  Each step shifts 4 new
  bits in, so consecutive pairs share Q - 4 bits (a bitshift trellis with a Q-bit state).
* The pair's value is a 2-D codebook vector: (w[2i], w[2i+1]) = (cb[state][0], cb[state][1]),
  from a 2**Q x 2 table of fp16 values, Q = 9 (a 2 KiB table: the whole decoder is a lookup
  table, which is what sets the rung apart from the bitshift rung's 2**16-entry one).
* Rounding as declared for the path: the fp16 codebook value is narrowed to bf16 (nearest-even),
  the dot product accumulates wide and the fp16 per-output-row scale multiplies it afterwards.
* Storage: the bitshift rung's block-interleaved layout (oracle.trellis.stored_rows, here
  stored_rows too, turns stored bytes back into the rows above); every decode below takes rows.
"""
from __future__ import annotations

import numpy as np

from . import trellis

LUT_RUNG_BITS = 9            # Q: codebook index bits
STEP_BITS = 4                # bits a step consumes: 2 weights x 2 bits


stored_rows = trellis.stored_rows  # both rungs store their matrices the same way


def pair_state_bruteforce(row_bytes, i: int, q: int = LUT_RUNG_BITS) -> int:
    """State of pair i of one row, bit by bit: the q stream bits from bit 4i on, circular."""
    nbits = 8 * len(row_bytes)
    s = 0
    for b in range(q):
        pos = (STEP_BITS * i + b) % nbits
        bit = (int(row_bytes[pos // 8]) >> (pos % 8)) & 1
        s += bit << b
    return s


def pair_states(codes: np.ndarray, q: int = LUT_RUNG_BITS) -> np.ndarray:
    """codes [..., cols/4] uint8 -> pair states [..., cols/2] (int64), vectorised from the definition."""
    c = np.asarray(codes, dtype=np.uint8)
    bits = np.unpackbits(c, axis=-1, bitorder="little")        # [..., 2*cols], bit j of the stream
    nbits = bits.shape[-1]
    starts = np.arange(0, nbits, STEP_BITS)
    state = np.zeros(bits.shape[:-1] + (starts.size,), np.int64)
    for b in range(q):
        state += bits[..., (starts + b) % nbits].astype(np.int64) << b
    return state


def codebook_bf16(codebook_f16: np.ndarray) -> np.ndarray:
    """The codebook [2**Q, 2] narrowed to bf16 (fp16 -> exact fp32 -> bf16 nearest-even), as float64."""
    from .numerics import bf16_round
    return bf16_round(np.asarray(codebook_f16, dtype=np.float16).astype(np.float32))


def decode_declared(codes: np.ndarray, codebook_f16: np.ndarray, q: int = LUT_RUNG_BITS) -> np.ndarray:
    """Unscaled weights [..., rows, cols] in the declared precision: bf16 codebook values, float64."""
    cb = codebook_bf16(codebook_f16)
    st = pair_states(codes, q)
    w = cb[st]                                   # [..., rows, cols/2, 2]
    return w.reshape(*w.shape[:-2], w.shape[-2] * 2)


def decode_exact(codes: np.ndarray, codebook_f16: np.ndarray, scales_f16: np.ndarray,
                 q: int = LUT_RUNG_BITS) -> np.ndarray:
    """Scaled weights with no narrowing: float32(codebook) * float32(scale[row]) as float64."""
    cb = np.asarray(codebook_f16, dtype=np.float16).astype(np.float64)
    w = cb[pair_states(codes, q)]
    w = w.reshape(*w.shape[:-2], w.shape[-2] * 2)
    return w * np.asarray(scales_f16, dtype=np.float16).astype(np.float64)[..., :, None]


def dense_weights_bruteforce(codes_2d, codebook_f16, scales_f16=None, declared=True,
                             q: int = LUT_RUNG_BITS) -> np.ndarray:
    """One matrix's weights element by element (pure Python loops over rows and pairs)."""
    from .numerics import bf16_round
    cb = np.asarray(codebook_f16, dtype=np.float16).astype(np.float64)
    rows = codes_2d.shape[0]
    cols = 4 * codes_2d.shape[1]
    out = np.zeros((rows, cols), np.float64)
    for r in range(rows):
        for i in range(cols // 2):
            s = pair_state_bruteforce(codes_2d[r], i, q)
            for half in range(2):
                v = cb[s][half]
                if declared:
                    out[r, 2 * i + half] = float(bf16_round(v))
                else:
                    out[r, 2 * i + half] = float(np.float32(v)) * float(np.float32(scales_f16[r]))
    return out
