"""Build libjsverify.so (HIP, gfx950) in-tree with hipcc.

    python -m draft_block_verification_rmsnorm_amd.build      # or build() from Python
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libjsverify.so"
SOURCES = [CSRC / "jsv_api.hip", CSRC / "jsv_kernels.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep hand-written fp32 arithmetic off the packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libjsverify")


def build(verbose: bool = False, extra_flags=None) -> Path:
    """Compile every HIP source into PKG/libjsverify.so; returns the library path."""
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", str(INCLUDE), "-I", str(CSRC),
           *map(str, SOURCES), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    print(LIB)
