"""The host-side ABI tests (argument validation, size and workspace queries, codebook
tables) run again against a build of the library whose host code is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer.  No GPU: every call in those tests
returns before any launch."""
import os
import subprocess
import sys

import pytest

from bit_nf4_quantized_11_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    for cc in ("/opt/rocm/llvm/bin/clang", "clang"):
        try:
            out = subprocess.run([cc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                                 text=True, timeout=60).stdout.strip()
        except (OSError, subprocess.TimeoutExpired):
            continue
        if out and os.path.isabs(out) and os.path.exists(out):
            return out
    return None


def test_abi_under_address_and_ub_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = build.build(sanitize=True)
    env = dict(os.environ)
    env["QLORA_LIB"] = lib
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
