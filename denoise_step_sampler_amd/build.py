"""Builds libdg.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdg.so")
SOURCES = ["dg_api.hip", "vocab_gemm.hip", "embedding_f16.hip", "accept_renoise.hip", "q_sample.hip",
           "selfcond_ffw.hip", "lite_sampler.hip",
           "fp8.hip"]
HEADERS = ["dg_device.h", "dg_internal.h"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every source into libdg.so (always recompiles).  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(PKG, "..", "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libdg.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
