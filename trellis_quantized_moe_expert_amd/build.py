"""Build the HIP library libqtip_moe.so in-tree for gfx950.

    python -m trellis_quantized_moe_expert_amd.build

hipcc cross-compiles without a GPU.  Packed-FP32 instruction selection is disabled for
all device code (-packed-fp32-ops off).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["csrc/api.hip", "csrc/route.hip", "csrc/expert.hip", "csrc/router.hip"]
OUTPUT = os.path.join(_HERE, "libqtip_moe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found")


def command(output: str = OUTPUT) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *[os.path.join(_HERE, s) for s in SOURCES], "-o", output]


def build_library(verbose: bool = False) -> str:
    tmp = OUTPUT + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build_library(verbose=True))
