"""Builds libkda.so (the gfx950 HIP kernels and the C ABI) in place.

    python -m chunked_gated_delta_kda_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libkda.so"
SOURCES = ["kda_api.hip", "kda_prep.hip", "kda_recur.hip", "kda_decode.hip", "kda_split.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda)")


def build(verbose: bool = False, extra_flags=()) -> Path:
    """Compile every HIP source for gfx950 into PKG/libkda.so (atomic replace)."""
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=str(PKG))
    os.close(fd)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           # no packed fp32 VALU ops anywhere: plain float code only
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA results in VGPRs: the kernels convert and rescale their
           # accumulators on the VALU every chunk, so AGPR round trips would cost
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           f"-I{INCLUDE}", f"-I{CSRC}", *extra_flags,
           *[str(CSRC / s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"libkda build failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    out = build(verbose=True)
    print(f"built {out}", file=sys.stderr)
