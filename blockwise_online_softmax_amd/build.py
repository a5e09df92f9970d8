"""Build libra.so (the HIP kernels and the C ABI) for gfx950 with hipcc, and
libra_probe.so (bench.py's MFMA-ceiling and clock probe, not part of the ABI).

Usage: python -m blockwise_online_softmax_amd.build   (or __graft_entry__.build())
The libraries are written next to this file; nothing is installed.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libra.so")
PROBE_LIB = os.path.join(HERE, "libra_probe.so")
PROBE_SOURCE = "ra_probe.hip"

SOURCES = ["ra_api.cpp", "ra_aux.hip", "ra_attn_valu.hip", "ra_attn_mfma.hip", "ra_merge.hip",
           "ra_vocab_ce.hip", "ra_xcd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose=False, jobs=4):
    """Compile every source to an object in parallel, then link libra.so and
    libra_probe.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES + [PROBE_SOURCE]:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c"] + lang + [
            os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag: harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln
                 and "is not a recognized feature for this target" not in ln]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    for lib, lib_objs in ((LIB, objs[:-1]), (PROBE_LIB, objs[-1:])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + lib_objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
