"""Build libswa.so (HIP, gfx950) in-tree with hipcc.

    python -m sliding_window_gqa_amd.build

Every source is compiled for gfx950 only; the library is linked next to this
file, where the binding loads it.  Packed float32 VALU instructions are
disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libswa.so")

SOURCES = ["swa_api.cpp", "swa_write.hip", "swa_prefill.hip", "swa_decode.hip", "swa_debug.hip",
           "swa_noalloc.hip"]
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Per-source extra flags.  The prefill kernel keeps its matrix-instruction
# results (the output accumulators, which the rare softmax rescale multiplies
# with vector instructions) in VGPRs and lets the operands live in AGPRs.
EXTRA = {"swa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libswa)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libswa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_c_check(verbose)
    return LIB


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "swa_c_check.c")
C_CHECK = os.path.join(ROOT, "tests", "c_abi", "swa_c_check")


def build_c_check(verbose: bool = False) -> str:
    """Compile the plain-C caller of the ABI (tests/c_abi) with gcc against
    include/swa.h and the freshly linked libswa.so; returns its path."""
    rocm = os.path.dirname(os.path.dirname(_hipcc()))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(rocm, 'include')}", f"-I{os.path.join(ROOT, 'include')}", C_CHECK_SRC,
           f"-L{PKG}", "-lswa", f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../sliding_window_gqa_amd", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
           "-o", C_CHECK]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {C_CHECK_SRC}:\n{r.stdout}\n{r.stderr}")
    return C_CHECK


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
