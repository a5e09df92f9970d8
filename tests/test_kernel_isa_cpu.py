"""Register budget of the matrix-core attention kernel, checked on the CPU from
the gfx950 assembly that hipcc writes for it.

Two kinds of source change have moved the tile loop's walker (its block, tile
and position arithmetic, uniform across a wavefront) from scalar to vector
registers without any error: indexing a field of the kernel's parameter struct
by a runtime value, and a branch on the layout where the work item is decoded.
Either way the kernels reached the 104-106 scalar-register limit and the loop
grew by about 500 instructions.  This test compiles the kernel file and fails
if any instantiation needs more than 100 scalar registers, or if a ring kernel
(no state in HBM, no position arrays) uses scratch memory."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_online_softmax_amd", "csrc")


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else shutil.which("hipcc")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    out = tmp_path_factory.mktemp("isa") / "ra_attn_mfma.s"
    cmd = [hipcc, "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, "ra_attn_mfma.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    res, name = {}, None
    for line in open(out):
        m = re.match(r"^(_Z\S*attn_mfma_kernel\S*):", line)
        if m:
            name = m.group(1)
            res[name] = {}
            continue
        if name is None:
            continue
        for key in ("TotalNumSgprs", "NumVgprs", "ScratchSize"):
            m = re.match(rf"^\s*; {key}: (\d+)", line)
            if m:
                res[name][key] = int(m.group(1))
        if "ScratchSize" in res[name]:
            name = None
    assert len(res) >= 24, sorted(res)
    return res


def _template_args(name):
    """(D, NW, causal, pos mode, state in HBM, natural order) of a mangled name."""
    m = re.search(r"attn_mfma_kernelILi(\d+)ELi(\d+)ELb(\d)ELi(\d)ELb(\d)ELb(\d)E", name)
    assert m, name
    return tuple(int(x) for x in m.groups())


def test_scalar_register_budget(kernels):
    over = {n: r["TotalNumSgprs"] for n, r in kernels.items() if r["TotalNumSgprs"] > 100}
    assert not over, over


def test_ring_kernels_use_no_scratch(kernels):
    ring = {n: r for n, r in kernels.items()
            if _template_args(n)[4] == 0 and _template_args(n)[3] != 2}
    assert len(ring) >= 12
    spill = {n: r["ScratchSize"] for n, r in ring.items() if r["ScratchSize"] != 0}
    assert not spill, spill
