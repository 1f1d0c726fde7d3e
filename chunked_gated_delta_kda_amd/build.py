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
SOURCES = ["kda_api.hip", "kda_prep.hip", "kda_recur.hip", "kda_fused.hip", "kda_decode.hip",
           "kda_split.hip", "kda_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda)")


# Sources whose kernels keep MFMA results in VGPRs rather than AGPRs.  The
# backward gradient kernel is left to the compiler's default: its register
# demand exceeds the VGPR file, and the VGPR-form rewrite crashes on it.
VGPR_FORM = {"kda_api.hip", "kda_prep.hip", "kda_recur.hip", "kda_fused.hip", "kda_decode.hip",
             "kda_split.hip"}


# Sources scheduled with the compiler's iterative ILP strategy instead of the
# default occupancy-driven one (same results, bit for bit): the single-launch
# kernel's SIMDs are issue-bound with two waves each, and it measured 2-2.5%
# faster on every workload; the chunk-preparation kernel 3.6% faster.  On the
# recurrence, split and gradient kernels it measured within the spread.
ILP_SCHED = {"kda_fused.hip", "kda_prep.hip"}


def source_flags(src: str) -> list:
    """The code-generation flags of one source (beyond the common ones)."""
    flags = []
    if src in VGPR_FORM:
        # MFMA results in VGPRs: the kernels convert and rescale their
        # accumulators on the VALU every chunk, so AGPR round trips would cost
        flags += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    if src in ILP_SCHED:
        flags += ["-mllvm", "--amdgpu-sched-strategy=iterative-ilp"]
    return flags


def _compile(src: str, obj: Path, extra_flags) -> subprocess.CompletedProcess:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
           "-Wall", "-Wno-unused-function",
           # no packed fp32 VALU ops anywhere: plain float code only
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{INCLUDE}", f"-I{CSRC}", *extra_flags, *source_flags(src)]
    cmd += [str(CSRC / src), "-o", str(obj)]
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, extra_flags=()) -> Path:
    """Compile every HIP source for gfx950 (in parallel) and link PKG/libkda.so
    (atomic replace)."""
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory(dir=str(PKG)) as td:
        objs = [Path(td) / (Path(s).stem + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            results = list(ex.map(lambda so: _compile(so[0], so[1], extra_flags),
                                  zip(SOURCES, objs)))
        for src, res in zip(SOURCES, results):
            if verbose:
                print(" ".join(res.args), flush=True)
            if res.returncode != 0:
                raise RuntimeError(f"libkda build failed ({src}):\n{res.stderr}")
        fd, tmp = tempfile.mkstemp(suffix=".so", dir=str(PKG))
        os.close(fd)
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            os.unlink(tmp)
            raise RuntimeError(f"libkda link failed:\n{res.stderr}")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    out = build(verbose=True)
    print(f"built {out}", file=sys.stderr)
