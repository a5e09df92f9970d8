"""A build of libra.so with AddressSanitizer and UndefinedBehaviorSanitizer on
the host side: the C-ABI layer, argument validation, the XCD planner and
every other piece of host C++.  Device code is compiled as usual (no
sanitizer: the flags reach only the host pass).  For CPU tests of the ABI's
error paths; the library is never used on a GPU.

Usage: python -m blockwise_online_softmax_amd.build_sanitized
Writes _build_san/libra_san.so next to this file and prints its path.  Load it
with the sanitizer runtime preloaded (asan_runtime() gives its path).
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from .build import CSRC, INCLUDE, SOURCES, hipcc

HERE = os.path.dirname(os.path.abspath(__file__))
OUT_DIR = os.path.join(HERE, "_build_san")
LIB = os.path.join(OUT_DIR, "libra_san.so")

# each sanitizer flag directly after -Xarch_host: host code only
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def asan_runtime():
    """Path of the ROCm clang's shared AddressSanitizer runtime (None if absent)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build(jobs=4):
    os.makedirs(OUT_DIR, exist_ok=True)

    def one(src):
        obj = os.path.join(OUT_DIR, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc()] + FLAGS + SAN_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c"] + lang + [
            os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-3000:]}")
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.stdout.flush()
