"""Build libkivi.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Every call recompiles.  Usage: ``python -m decode_attention_pack_amd.build``.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkivi.so")
OBJDIR = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "pack.hip", "decode_generic.hip", "decode_vector.hip", "decode_matrix.hip",
           "select.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-x", "hip",
    # keep the compiler away from packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every rounding step as written: no implicit fusion of a multiply with an
    # add or a narrowing conversion (kernels call fmaf where they want one)
    "-ffp-contract=off",
    # a work-counter draw by one lane stays one atomic whose result is read
    # where the kernel reads it (the atomic optimizer would read it back at
    # once, waiting for every memory operation in flight)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line
                     and line.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build() -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
