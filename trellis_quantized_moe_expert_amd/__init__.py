"""MI355X (gfx950) trellis-quantized MoE expert matmul.

The compute path is the HIP library libqtip_moe.so (C ABI in include/qtip_moe.h); this
package holds its sources (csrc/), the build script and a thin ctypes binding whose
functions carry the C names.  PyTorch provides device memory and streams only.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import lib, LIB_PATH, QtipError  # noqa: F401
