"""Build libdomino.so (HIP, gfx950) in-tree with hipcc.

    python -m draft_block_causal_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdomino.so")
SOURCES = ["kernels.hip", "rowstream.hip", "gemm.hip", "loop.hip", "loop_b1.hip", "verify.hip", "base_draft.hip", "loss.hip", "backward.hip", "gru_backward.hip",
           "api.cpp", "validate.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
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


def build(verbose: bool = False) -> str:
    """Compile every HIP source into draft_block_causal_amd/libdomino.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
