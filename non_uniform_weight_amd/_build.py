"""Build step of the package: compiles libsqllm.so (HIP, gfx950) in-tree.

Run it by path (``python non_uniform_weight_amd/_build.py``): importing it as
``non_uniform_weight_amd._build`` would first import the package, which
refuses to load without the library."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsqllm.so")

SOURCES = ["sqllm_fused2.hip", "sqllm_gemv2.hip", "sqllm_fused3.hip", "sqllm_fused3c.hip", "sqllm_fused4.hip", "sqllm_gemv3.hip",
           "sqllm_gemv4.hip", "sqllm_wide2.hip", "sqllm_wide3.hip", "sqllm_wide4.hip", "sqllm_sparse.hip",
           "sqllm_pack.hip", "sqllm_quantize.hip", "sqllm_noalloc.hip", "sqllm_api.cpp"]
OBJDIR = os.path.join(PKG, "_build")

# gfx950 only; packed fp32 instructions are switched off (the device pass
# honours the feature, the host pass warns that it does not know it).
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function"]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libsqllm.so")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if ln.strip() and NOISE not in ln]
    if proc.returncode != 0:
        raise RuntimeError(f"{os.path.basename(cmd[-1])}: hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose: bool = False, extra_flags: list[str] | None = None, jobs: int = 0) -> str:
    """Compile every source to an object in parallel, then link libsqllm.so
    next to this file."""
    os.makedirs(OBJDIR, exist_ok=True)
    flags = [*HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC]
    objs = [os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    cmds = [[hipcc(), *flags, "-c", "-o", obj, os.path.join(CSRC, src)] for src, obj in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for fut in [pool.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
