"""Build the gfx950 MLA decode library in-tree with hipcc.

``python -m decode_attention_mla_amd.build`` (or ``build()``) always
recompiles every source under ``csrc/`` into ``_lib/libmla_decode.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "mla_kernels.hip")         # the attention kernels
STEPS_SRC = os.path.join(PKG, "csrc", "mla_steps.hip")     # the MLA steps around them
API_SRC = os.path.join(PKG, "csrc", "mla_api.cpp")         # host side of the C ABI
NOALLOC_SRC = os.path.join(PKG, "csrc", "mla_noalloc.hip")  # the entry point that allocates nothing
SRCS = [SRC, STEPS_SRC, API_SRC, NOALLOC_SRC]              # every source of the library
LIB = os.path.join(PKG, "_lib", "libmla_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in vector registers: the kernels scale them with
    # vector ALU (softmax rescale), which cannot read accumulation registers
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(PKG, "csrc"),
]


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
