"""Build libkron.so in-tree with hipcc for gfx950.

    python -m kronecker_factored_structured_amd.build

Every HIP source under csrc/ and the C-ABI layer are compiled into one shared library
next to this file.  Packed-FP32 instruction selection is disabled for the device code
(see the flag list); no fast-math flags are used, so fp32 results follow IEEE rounding
of each operation.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkron.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "kron_api.cpp",
    "kron_generic.hip",
    "kron_mfma.hip",
    "ks_matmul.hip",
    "ks_mfma.hip",
    "adam_l1.hip",
    "head_ce.hip",
]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-cuda-compat",
    "-I", INCLUDE, "-I", CSRC,
]


def command(out: str = LIB) -> list:
    srcs = []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        srcs += (["-x", "hip", path] if s.endswith(".cpp") else [path])
    return [HIPCC] + FLAGS + srcs + ["-o", out]


def build(verbose: bool = False) -> str:
    """Compile libkron.so (always recompiles) and return its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
