"""Build the gfx950 shared library libmi355_attn.so in-tree with hipcc (no GPU needed: hipcc cross-compiles).

    python -m transformer_head_scaled_02_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libmi355_attn.so"

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax rescales them with VALU ops, which cannot address AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # no NaN inputs are supported (they are not valid attention inputs): fmaxf then maps directly onto v_max3_f32
    # without canonicalising its operands
    "-fno-honor-nans",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(CSRC.glob("*.hip"))


def build_library(verbose: bool = False) -> Path:
    """Compile every HIP source for gfx950 and link libmi355_attn.so next to this file. Always rebuilds."""
    hipcc = _hipcc()
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    objs = [BUILD / (s.stem + ".o") for s in srcs]

    def compile_one(src_obj):
        src, obj = src_obj
        cmd = [hipcc, *HIP_FLAGS, "-c", str(src), "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src.name}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
