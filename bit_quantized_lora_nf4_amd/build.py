"""Compile the HIP library ``libqlora_nf4.so`` for gfx950 with hipcc (in-tree).

Usage: ``python -m bit_quantized_lora_nf4_amd.build`` (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the shared library is written
next to this file.  Every call recompiles.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqlora_nf4.so")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Strict IEEE fp32 where the decode must be bit-exact: no contraction of a*b+c into
# fma unless written as fma, correctly rounded division, denormals preserved.
# Packed fp32 instructions are disabled for all device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]

SOURCES = ["codebook.cpp", "api.cpp", "quantize.hip", "dequant.hip", "lora.hip", "gemm.hip", "adamw.hip", "merge.hip",
           "gemv.hip"]


def _compile(src, obj_dir, verbose):
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose=False, jobs=None):
    """Compile every source and link ``libqlora_nf4.so``; returns its path."""
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
