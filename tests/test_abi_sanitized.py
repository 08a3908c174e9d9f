"""The C-ABI argument checks under AddressSanitizer and UndefinedBehaviorSanitizer (host code only; no GPU needed).

The library is rebuilt with -fsanitize=address,undefined on its host compilation (the gfx950 device code is that of
the normal build) and the whole CPU ABI suite, tests/test_abi_cpu.py, runs against it in a child process with the
ASan runtime preloaded. Every rejected call there walks the validation code (null pointers, sizes, overlaps,
workspace limits, error strings) without a device, so an out-of-bounds access, a use after free, a signed overflow or
a misaligned load in that code fails the run."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

from transformer_head_scaled_02_amd import build

ROOT = Path(__file__).resolve().parents[1]

pytestmark = pytest.mark.skipif(not Path("/opt/rocm/bin/hipcc").exists(), reason="hipcc is needed to build")


@pytest.fixture(scope="module")
def sanitized_lib():
    lib = build.SANITIZED_LIB
    newest = max(p.stat().st_mtime for p in [*build.CSRC.iterdir(), Path(build.__file__)])
    if not lib.exists() or lib.stat().st_mtime < newest:
        build.build_library(sanitize=True)
    return lib


def _env(lib):
    env = dict(os.environ)
    env["MI355_ATTN_LIB"] = str(lib)
    env["LD_PRELOAD"] = ":".join(build.sanitizer_runtimes() + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    # CPython itself is not instrumented and keeps allocations alive at exit: leak reports would be its own
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    return env


def test_sanitized_build_is_instrumented(sanitized_lib):
    syms = subprocess.run(["nm", "-D", "--undefined-only", str(sanitized_lib)], capture_output=True, text=True,
                          check=True).stdout
    assert "__asan_report_load" in syms or "__asan_load" in syms
    assert "__ubsan_handle_" in syms


def test_runtime_is_active_in_the_child(sanitized_lib):
    code = ("import ctypes, transformer_head_scaled_02_amd as m; lib = m.load_library(); "
            "ctypes.CDLL(None)['__asan_init']; print(m.LIB_PATH); "
            "print(lib.sdpa_forward(None, None, None, 0, None, 1, 1, 1, 1, 1, 64, 64, None))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(sanitized_lib), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = r.stdout.split()
    assert lines[0] == str(sanitized_lib) and lines[1] == "1"  # ATTN_ERR_INVALID from the sanitized library


def test_abi_suite_under_asan_and_ubsan(sanitized_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi_cpu.py"],
                       cwd=ROOT, env=_env(sanitized_lib), capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
