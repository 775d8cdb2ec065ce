"""Build libkron.so in-tree with hipcc for gfx950.

    python -m kronecker_factored_structured_amd.build

Every HIP source under csrc/ and the C-ABI layer are compiled to objects (in parallel)
and linked into one shared library next to this file.  Packed-FP32 instruction selection is disabled for the device code
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

# (source, extra flags, object name): kron_mfma.hip is compiled twice, its forward kernels
# with LLVM's instruction-level-parallelism scheduler (measured faster for them) and the
# rest with the default one.
OBJECTS = [
    ("kron_api.cpp", [], "kron_api"),
    ("kron_generic.hip", [], "kron_generic"),
    ("kron_mfma.hip", ["-DKRON_MFMA_PASS=1", "-mllvm", "-amdgpu-sched-strategy=max-ilp"], "kron_mfma_fwd"),
    ("kron_mfma.hip", ["-DKRON_MFMA_PASS=2"], "kron_mfma_bwd"),
    ("kron_small.hip", [], "kron_small"),
    ("kron_bf16.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"], "kron_bf16"),
    ("ks_matmul.hip", [], "ks_matmul"),
    ("ks_mfma.hip", [], "ks_mfma"),
    ("ks_bwd.hip", [], "ks_bwd"),
    ("ks_chain.hip", [], "ks_chain"),
    ("vanloan.hip", [], "vanloan"),
    ("adam_l1.hip", [], "adam_l1"),
    ("head_ce.hip", [], "head_ce"),
    ("loss_terms.hip", [], "loss_terms"),
]
SOURCES = sorted({src for src, _, _ in OBJECTS})

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-cuda-compat",
    "-I", INCLUDE, "-I", CSRC,
]


# Host-only AddressSanitizer and UndefinedBehaviorSanitizer (each flag behind -Xarch_host,
# so no device code is instrumented): a build of the library for checking the host side,
# the argument validation of the C ABI above all, on the CPU.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def compile_commands(objdir: str, host_sanitize: bool = False) -> list:
    cmds = []
    for src, extra, name in OBJECTS:
        path = os.path.join(CSRC, src)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        san = HOST_SANITIZE if host_sanitize else []
        cmds.append([HIPCC] + FLAGS + extra + san + ["-c"] + lang + [path, "-o", os.path.join(objdir, name + ".o")])
    return cmds


def link_command(objdir: str, out: str, host_sanitize: bool = False) -> list:
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"] \
        if host_sanitize else []
    return [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + \
        [os.path.join(objdir, name + ".o") for _, _, name in OBJECTS] + san + ["-o", out]


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload into a process that
    loads the host-sanitized library), or '' when it is not installed."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else ""


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd[-3:])}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)


def build(verbose: bool = False, host_sanitize: bool = False, out: str = LIB) -> str:
    """Compile libkron.so (always recompiles) to `out` and return its path."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    with tempfile.TemporaryDirectory(prefix="kron_build_") as objdir:
        cmds = compile_commands(objdir, host_sanitize)
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = out + ".tmp"
        _run(link_command(objdir, tmp, host_sanitize), verbose)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    # python -m kronecker_factored_structured_amd.build [--host-sanitize OUT.so]
    if len(sys.argv) == 3 and sys.argv[1] == "--host-sanitize":
        print(build(verbose=True, host_sanitize=True, out=os.path.abspath(sys.argv[2])))
    else:
        print(build(verbose=True))
