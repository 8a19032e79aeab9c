"""CPU oracle for the trellis-quantized MoE expert matmul (TEST INFRASTRUCTURE ONLY).

A plain, slow, obviously-correct numpy implementation of what the GPU path
computes, written from the source pages and checked against pins that do not come
from itself (tests/test_oracle_*.py).  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product library never does, and
shares no code, constants or helpers with it.  Floating point is evaluated in
float64 except at the rounding points the path declares (bf16 LUT values, bf16
intermediate activation, final output cast), which are modelled explicitly.

Modules
  trellis  -- bitstream -> symbols -> 16-bit window state -> LUT value (decode, bitshift rung)
  lut_rung -- bitstream -> 9-bit pair state -> 2-D codebook vector (decode, LUT rung)
  pool     -- the layer over a process pool for large layers (scheduling only)
  routing  -- top-k routing, softmax over the selected logits, expert binning, m-tile map
  fill     -- the closed-form m-tile fill model and the grouped-arm dispatch predicate
  moe      -- one MoE layer: gated experts, weighted combine, and a separately written
              dense-dequantised reference
  numerics -- the oracle's own bf16 rounding

Parity pins: every function is pinned by tests/test_oracle_*.py; the one item
left "parity unpinned" is compatibility of the bit layouts (both rungs) with real
QTIP checkpoints (no checkpoint or encoder exists in these inputs).
"""
