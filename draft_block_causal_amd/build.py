"""Build libdomino.so (HIP, gfx950) in-tree with hipcc.

    python -m draft_block_causal_amd.build

Each source is compiled to its own object in parallel (objects under _build/
next to this file), then the objects are linked into the shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdomino.so")
OBJ_DIR = os.path.join(PKG, "_build")
SOURCES = ["kernels.hip", "rowstream.hip", "gemm.hip", "loop.hip", "loop_b1.hip", "loop_bn.hip", "verify.hip", "base_draft.hip",
           "loss.hip", "backward.hip", "gru_backward.hip", "noalloc.hip", "api.cpp", "validate.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 instructions stay off: the compiler must not form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the Domino engine needs ROCm's hipcc for gfx950")


def _jobs() -> int:
    n = os.cpu_count() or 1
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        v = os.environ.get(var)
        if v and v.isdigit():
            n = min(n, int(v))
    return max(1, min(n, 16))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into draft_block_causal_amd/libdomino.so (always recompiles)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} ({res.returncode}):\n{res.stdout}\n{res.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
