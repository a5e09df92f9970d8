"""The workloads at full size, in the launch configuration bench.py times,
against the oracle.

mha16k, gqa32k and the three gqa64k layouts are compared with O1 over every
element of out and lse (the oracle runs on a pool of CPU processes, causal
rows meeting only the keys they can see).  share1m, device 0's share of a
1M-token ring, is compared on 256 sampled rows: half from each zigzag chunk,
every chunk's first and last row included."""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
import workloads
from oracle import attention as O1
from oracle import layouts as OL
from oracle import parallel as OP
from gpu_helpers import TOL, log, maxerr, to_np

pytestmark = pytest.mark.gpu

N_ROWS = 256


def progress(done, total, sec):
    log(f"    oracle: {done}/{total} rows in {sec:.0f} s")


def oracle_whole(name, q, k, v, causal):
    log(f"  {name}: oracle over every row ({OP.default_workers()} worker processes)")
    ro, rl, info = OP.full_attention_pool(q, k, v, causal=causal, progress=progress)
    log(f"  {name}: oracle took {info['seconds']:.1f} s on {info['workers']} workers "
        f"({info['cpu_model']})")
    return ro, rl


def whole_check(name, out, lse, ro, rl):
    """Max-abs error over every element, one head at a time."""
    tol_o, tol_l = TOL[torch.bfloat16]
    eo = el = 0.0
    for h in range(out.shape[1]):
        eo = max(eo, maxerr(to_np(out[0, h]), ro[0, h]))
        el = max(el, maxerr(to_np(lse[0, h]), rl[0, h]))
    n = out.numel()
    log(f"  {name}: all {n} outputs and {lse.numel()} lse: max|out err| {eo:.3e} "
        f"(tol {tol_o}), max|lse err| {el:.3e} (tol {tol_l})")
    assert eo <= tol_o and el <= tol_l, (name, eo, el)


@pytest.mark.parametrize("name", ["mha16k", "gqa32k"])
def test_contiguous_workloads(name):
    w = workloads.WORKLOADS[name]
    log(f"{name}: generating inputs")
    q, k, v = workloads.workload_inputs(name)
    out, lse = ra.ring_attention(q.cuda(), k.cuda(), v.cuda(), w["N"], "contiguous", w["causal"])
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    torch.cuda.empty_cache()
    ro, rl = oracle_whole(name, q, k, v, w["causal"])
    whole_check(name, out, lse, ro, rl)


def test_gqa64k_layouts():
    """S = 65536 causal: contiguous, striped and zigzag rings on the same
    tensors (natural order in and out), each against one oracle result."""
    w = workloads.WORKLOADS["gqa64k"]
    log("gqa64k: generating inputs")
    q, k, v = workloads.workload_inputs("gqa64k")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    res = {}
    for layout in ("contiguous", "striped", "zigzag"):
        out, lse = ra.ring_attention(qd, kd, vd, w["N"], layout, True)
        torch.cuda.synchronize()
        res[layout] = (out.cpu(), lse.cpu())
        del out, lse
    del qd, kd, vd
    torch.cuda.empty_cache()
    ro, rl = oracle_whole("gqa64k", q, k, v, True)
    for layout, (out, lse) in res.items():
        whole_check(f"gqa64k {layout}", out, lse, ro, rl)


def test_share1m():
    """Device 0's zigzag share of a 1,048,576-token ring: 131072 queries against
    all 8 key/value blocks in device order; 256 sampled rows, half from each
    zigzag chunk, every chunk's first and last row included."""
    w = workloads.WORKLOADS["share1m"]
    S, N = w["S"], w["N"]
    log("share1m: generating inputs")
    q, k, v = workloads.workload_inputs("share1m")
    out, lse = ra.ring_attention(q.cuda(), k.cuda(), v.cuda(), N, "zigzag", True, device=0)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(lse).all() and torch.isfinite(out.float()).all()
    c = S // (2 * N)
    q_pos = OL.device_positions(S, N, "zigzag", 0)
    k_pos = OL.permuted_positions(S, N, "zigzag")
    Hq, Sq = q.shape[1], q.shape[2]
    rows = workloads.sample_rows(Hq, Sq, N_ROWS // Hq, seed=77, strata=[(0, c), (c, 2 * c)],
                                 include_ends=True)
    ro, rl = O1.attention_rows(q, k, v, [(0, h, i) for h, i in rows], q_pos=q_pos, k_pos=k_pos,
                               causal=True)
    go = np.stack([to_np(out[0, h, i]) for h, i in rows])
    gl = np.array([float(lse[0, h, i]) for h, i in rows])
    eo, el = maxerr(go, ro), maxerr(gl, rl)
    tol_o, tol_l = TOL[torch.bfloat16]
    log(f"  share1m: {len(rows)} sampled rows: max|out err| {eo:.3e}, max|lse err| {el:.3e}")
    assert eo <= tol_o and el <= tol_l, (eo, el)
