"""The C-ABI suite (tests/test_abi_cpu.py: every declared export, every error
path, the XCD planner, the layout map) run against a build of the library
whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer.
CPU only.  Any sanitizer report ends that run with a non-zero status."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from blockwise_online_softmax_amd import build_sanitized as bs

    rt = bs.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm installation")
    lib = bs.build()
    env = dict(os.environ)
    env.update({
        "RA_LIB": lib,
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-q", "-s", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    for marker in ("runtime error:", "ERROR: AddressSanitizer", "SUMMARY: "):
        assert marker not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out, out[-3000:]
