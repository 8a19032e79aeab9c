"""Build the HIP library libqtip_moe.so in-tree for gfx950.

    python -m trellis_quantized_moe_expert_amd.build

hipcc cross-compiles without a GPU.  Each source is compiled to an object on its own (in
parallel), keeping the gfx950 device assembly, and the objects are linked into one shared
library.

Packed FP32: every source is compiled with `-Xclang -target-feature -Xclang -packed-fp32-ops`,
which removes the packed-FP32 feature from the gfx950 device pass, so the compiler selects no
packed FP32 instructions (checked: a float2 multiply-add that compiles to packed FP32 without
the flag compiles to scalar VALU instructions with it).  hipcc also passes the flag to the x86
host pass, which prints that it does not know the feature and ignores it; that warning is
harmless.  After compiling, the build scans the device assembly and fails if any packed FP32
instruction appears, so the property is checked on every build, not assumed.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["csrc/api.hip", "csrc/route.hip", "csrc/expert.hip", "csrc/expert_lut.hip", "csrc/router.hip"]
OUTPUT = os.path.join(_HERE, "libqtip_moe.so")
BUILD_DIR = os.path.join(os.path.dirname(_HERE), "_build")
ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# packed FP32 arithmetic mnemonics (fma, add, mul on two fp32 lanes)
PACKED_FP32 = re.compile(r"\bv_pk_(fma|add|mul)_f32\b")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found")


def compile_command(src: str, obj: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", *DEVICE_FLAGS,
            "-save-temps=obj", "-c", os.path.join(_HERE, src), "-o", obj]


def link_command(objs: list, output: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", output]


def device_asm_files(obj_dir: str) -> list:
    return sorted(os.path.join(obj_dir, f) for f in os.listdir(obj_dir)
                  if f.endswith(".s") and f"amdgcn-amd-amdhsa-{ARCH}" in f)


def packed_fp32_lines(asm_text: str) -> list:
    """Lines of device assembly that hold a packed FP32 instruction."""
    return [ln.strip() for ln in asm_text.splitlines() if PACKED_FP32.search(ln.split(";")[0])]


def _compile(src: str) -> tuple:
    name = os.path.splitext(os.path.basename(src))[0]
    obj_dir = os.path.join(BUILD_DIR, name)
    os.makedirs(obj_dir, exist_ok=True)
    obj = os.path.join(obj_dir, name + ".o")
    cmd = compile_command(src, obj)
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=obj_dir)
    return src, obj, obj_dir, cmd, res


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for src, obj, obj_dir, cmd, res in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {src} with exit code {res.returncode}")
        asm = device_asm_files(obj_dir)
        if not asm:
            raise RuntimeError(f"no {ARCH} device assembly was kept for {src}")
        for path in asm:
            bad = packed_fp32_lines(open(path).read())
            if bad:
                raise RuntimeError(f"{src}: packed FP32 instructions in the device code: {bad[:4]}")
        objs.append(obj)
    tmp = OUTPUT + ".tmp"
    cmd = link_command(objs, tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build_library(verbose=True))
