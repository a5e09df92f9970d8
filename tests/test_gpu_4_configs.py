"""The workloads at full size, in the launch configuration bench.py times,
checked against the oracle on 256 seeded sampled rows each, plus properties
that hold at any size over the whole output (finite values, every output a
convex combination of value rows, layout invariance)."""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
import workloads
from oracle import attention as O1
from oracle import layouts as OL
from gpu_helpers import TOL, log, maxerr, to_np

pytestmark = pytest.mark.gpu

N_ROWS = 256


def sampled_check(name, q, k, v, out, lse, q_pos, k_pos, causal, strata=None):
    Hq, Sq = q.shape[1], q.shape[2]
    per_head = N_ROWS // Hq
    rows = workloads.sample_rows(Hq, Sq, per_head, seed=77, strata=strata,
                                 include_ends=strata is not None)
    ro, rl = O1.attention_rows(q, k, v, [(0, h, i) for h, i in rows], q_pos=q_pos, k_pos=k_pos,
                               causal=causal)
    go = np.stack([to_np(out[0, h, i]) for h, i in rows])
    gl = np.array([float(lse[0, h, i]) for h, i in rows])
    eo, el = maxerr(go, ro), maxerr(gl, rl)
    tol_o, tol_l = TOL[torch.bfloat16]
    log(f"  {name}: {len(rows)} sampled rows: max|out err| {eo:.3e}, max|lse err| {el:.3e}")
    assert eo <= tol_o and el <= tol_l, (eo, el)


def whole_output_checks(out, lse, v):
    assert torch.isfinite(lse).all(), "non-finite lse"
    assert torch.isfinite(out.float()).all(), "non-finite out"
    vmax = float(v.float().abs().max())
    assert float(out.float().abs().max()) <= vmax * (1 + 2 ** -7)


@pytest.mark.parametrize("name", ["mha16k", "gqa32k"])
def test_contiguous_workloads(name):
    w = workloads.WORKLOADS[name]
    log(f"{name}: generating inputs")
    q, k, v = workloads.workload_inputs(name)
    out, lse = ra.ring_attention(q.cuda(), k.cuda(), v.cuda(), w["N"], "contiguous", w["causal"])
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    whole_output_checks(out, lse, v)
    sampled_check(name, q, k, v, out, lse, None, None, w["causal"])


def test_gqa64k_layouts():
    """S = 65536 causal: contiguous, striped and zigzag rings on the same
    tensors, each against the oracle on sampled rows and against each other
    over the whole output."""
    w = workloads.WORKLOADS["gqa64k"]
    log("gqa64k: generating inputs")
    q, k, v = workloads.workload_inputs("gqa64k")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    base = None
    for layout in ("contiguous", "striped", "zigzag"):
        out, lse = ra.ring_attention(qd, kd, vd, w["N"], layout, True)
        torch.cuda.synchronize()
        oc, lc = out.cpu(), lse.cpu()
        whole_output_checks(oc, lc, v)
        sampled_check(f"gqa64k {layout}", q, k, v, oc, lc, None, None, True)
        if base is None:
            base = (out, lse)
        else:
            eo = float((out.float() - base[0].float()).abs().max())
            el = float((lse - base[1]).abs().max())
            log(f"  {layout} vs contiguous over the whole output: out {eo:.2e} lse {el:.2e}")
            assert eo <= 2e-2 and el <= 1e-3
        del out, lse


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
    whole_output_checks(out, lse, v)
    c = S // (2 * N)
    q_pos = OL.device_positions(S, N, "zigzag", 0)
    k_pos = OL.permuted_positions(S, N, "zigzag")
    sampled_check("share1m", q, k, v, out, lse, q_pos, k_pos, True,
                  strata=[(0, c), (c, 2 * c)])
