"""Build libqlora.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m bit_nf4_quantized_11_amd.build [--jobs N] [--verbose] [--sanitize]

The library's version string carries a hash of every source it is built from (the
C/HIP sources, the public header and the compiler flags); the loader refuses a
library whose hash differs from the sources next to it.  --sanitize builds a
separate copy (_build/asan/libqlora.so) whose host code is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (device code is built as usual),
for running the host-side validation tests on the CPU.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqlora.so")

ARCH = os.environ.get("QLORA_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # bit-exact quantize/dequant paths: never fuse a*b+c unless written as fma
    "-ffp-contract=off",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
DEVICE = [
    f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# host-only instrumentation for the sanitizer build (each flag applies to the host pass only)
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libqlora.so")


def source_hash() -> str:
    """sha256 (first 16 hex digits) over the library's sources, its public header and the
    compile flags: the identity a built library is checked against when it is loaded."""
    h = hashlib.sha256()
    files = sources() + [os.path.join(INCLUDE, "qlora.h")] + sorted(
        os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    for path in files:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(COMMON[:-2] + DEVICE).encode())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libqlora")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool, out_dir: str = BUILD_DIR, sanitize: bool = False, tag: str = "") -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    extra = [f'-DQLORA_SOURCE_HASH="{tag}"'] if tag else []
    if src.endswith(".hip"):
        san = [f for flag in SANITIZE for f in ("-Xarch_host", flag)] if sanitize else []
        cmd = [hipcc(), "-x", "hip", *DEVICE, *COMMON, *extra, *san, "-c", src, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, *extra, *(SANITIZE if sanitize else []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def build(jobs: int | None = None, verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP/C++ source of the library and link libqlora.so into the package
    (or, with sanitize, the instrumented copy under _build/asan)."""
    out_dir = ASAN_DIR if sanitize else BUILD_DIR
    lib = ASAN_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    tag = source_hash()
    jobs = jobs or min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, sanitize, tag), srcs))
    tmp = lib + ".tmp"
    san = ["-fsanitize=address", "-fsanitize=undefined", "-shared-libsan"] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, a.sanitize))


if __name__ == "__main__":
    sys.exit(main())
