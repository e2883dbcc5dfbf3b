"""The C entry points' host-side argument handling under AddressSanitizer and
UndefinedBehaviorSanitizer, without a GPU.

The ABI tests (test_abi.py) run in a child process against libkvc_asan.so:
the same sources with the host pass sanitized (``python -m
kv_cached_gqa_attention_amd.build --sanitize``), the shared sanitizer runtime
preloaded ahead of whatever the environment already preloads. Any report
aborts the child. Skipped when that library is missing or older than the
sources, or the runtime is not installed.
"""

import os
import subprocess
import sys

import pytest

from kv_cached_gqa_attention_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def _stale(lib: str) -> bool:
    t = os.path.getmtime(lib)
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)]
    srcs.append(os.path.join(build.INCLUDE, "kvc.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


def test_abi_under_host_sanitizers():
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no shared AddressSanitizer runtime in the toolchain")
    if not os.path.exists(build.LIB_ASAN) or _stale(build.LIB_ASAN):
        pytest.skip("libkvc_asan.so missing or older than the sources: "
                    "python -m kv_cached_gqa_attention_amd.build --sanitize")
    env = dict(os.environ)
    env["KVC_LIB"] = build.LIB_ASAN
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "passed" in r.stdout
