"""Build the gfx950 shared library libmi355_attn.so in-tree with hipcc (no GPU needed: hipcc cross-compiles).

    python -m transformer_head_scaled_02_amd.build              # the library
    python -m transformer_head_scaled_02_amd.build --sanitize   # host-sanitized copy under _build/sanitized/
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


# Host-side sanitizers for the checking build: every -fsanitize= is given to the host compilation only
# (-Xarch_host), so the gfx950 device code is exactly that of the normal build.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]
SANITIZED_LIB = BUILD / "sanitized" / "libmi355_attn.so"


def sanitizer_runtimes() -> list[str]:
    """The clang ASan and UBSan runtimes matching hipcc, to preload into a process that loads the sanitized build."""
    roots = sorted(Path("/opt/rocm/llvm/lib/clang").glob("*/lib/linux"))
    for r in reversed(roots):
        asan, ubsan = r / "libclang_rt.asan-x86_64.so", r / "libclang_rt.ubsan_standalone-x86_64.so"
        if asan.exists():
            return [str(asan)]  # the ASan runtime carries the UBSan handlers as well
        if ubsan.exists():
            return [str(ubsan)]
    raise RuntimeError("clang sanitizer runtimes not found under /opt/rocm/llvm/lib/clang")


def build_library(verbose: bool = False, sanitize: bool = False) -> Path:
    """Compile every HIP source for gfx950 and link libmi355_attn.so next to this file. Always rebuilds.
    sanitize=True builds the host code with AddressSanitizer and UndefinedBehaviorSanitizer instead (device code
    unchanged) into _build/sanitized/libmi355_attn.so, for CPU-side argument-checking tests; the package's own library
    is left alone."""
    hipcc = _hipcc()
    out_dir = SANITIZED_LIB.parent if sanitize else BUILD
    out_dir.mkdir(parents=True, exist_ok=True)
    srcs = sources()
    objs = [out_dir / (s.stem + ".o") for s in srcs]
    extra = SANITIZE_FLAGS if sanitize else []

    def compile_one(src_obj):
        src, obj = src_obj
        cmd = [hipcc, *HIP_FLAGS, *extra, "-c", str(src), "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src.name}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    target = SANITIZED_LIB if sanitize else LIB
    tmp = target.with_suffix(".so.tmp")
    link_extra = ["-fsanitize=address,undefined", "-shared-libsan"] if sanitize else []
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, target)
    if verbose:
        print(f"built {target}")
    return target


if __name__ == "__main__":
    build_library(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
