"""Build ``libkvc.so`` (the C-ABI library) from ``csrc/`` with hipcc for gfx950.

Usage: ``python -m kv_cached_gqa_attention_amd.build`` (or ``build()`` from
Python). Always recompiles. Object files go to ``_build/`` beside this file;
the library lands next to this file, where the binding loads it from.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvc.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 instructions are disabled for all device code (the compiler
# would otherwise form v_pk_* from ordinary float code).
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


# Host-side sanitizers for a separate CPU-only check of the C entry points'
# argument handling (libkvc_asan.so): each sanitizer flag applies to the host
# pass only; device code is built as usual.
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()
LIB_ASAN = os.path.join(HERE, "libkvc_asan.so")
BUILD_ASAN = os.path.join(HERE, "_build_asan")
LLVM_BIN = os.environ.get("KVC_LLVM_BIN", "/opt/rocm/llvm/bin")


def asan_runtime() -> str | None:
    """The shared AddressSanitizer runtime of the ROCm clang (to preload into
    a process that loads libkvc_asan.so), or None."""
    import glob

    hits = sorted(glob.glob(os.path.join(os.path.dirname(LLVM_BIN), "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_ASAN if sanitize else BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


def build_sanitized(verbose: bool = True) -> str:
    """libkvc_asan.so: every source with the host pass under AddressSanitizer
    and UndefinedBehaviorSanitizer, linked against the shared sanitizer
    runtime. For CPU-side checks only (the GPU path loads libkvc.so)."""
    os.makedirs(BUILD_ASAN, exist_ok=True)
    srcs = _sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda x: _compile(x, True), srcs))
    tmp = LIB_ASAN + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
           *SAN_FLAGS, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_ASAN)
    if verbose:
        print(f"built {LIB_ASAN} from {len(srcs)} sources", file=sys.stderr)
    return LIB_ASAN


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build_sanitized()
    else:
        build()
