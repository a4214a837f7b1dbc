"""Build step of the package: compiles libsqllm.so (HIP, gfx950) in-tree.

Run it by path (``python non_uniform_weight_amd/_build.py``): importing it as
``non_uniform_weight_amd._build`` would first import the package, which
refuses to load without the library."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsqllm.so")

SOURCES = ["sqllm_kernels.hip", "sqllm_api.cpp"]

# gfx950 only; packed fp32 instructions are switched off (the device pass
# honours the feature, the host pass warns that it does not know it).
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libsqllm.so")
    return exe


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every HIP source into libsqllm.so next to this file."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if ln.strip() and noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
