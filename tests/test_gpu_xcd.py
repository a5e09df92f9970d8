"""The work split of ra_ring over the GPU's 8 XCDs.  A split moves whole work
items between XCDs, and every item is computed the same way wherever it runs,
so results under any split must be bit-identical to the fixed split; they are
also checked against the fp64 oracle on sampled rows.  The split launch is
also captured in a HIP graph and replayed.  Last, with measuring on, the speed
estimate must come from real measurements and stay plausible."""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
from oracle import attention as O1
from oracle import layouts as OL
from gpu_helpers import check, log, rand

pytestmark = pytest.mark.gpu

SKEW = [0.8, 1.2, 1.0, 1.0, 0.9, 1.1, 1.0, 1.0]


def _same(a, b):
    return torch.equal(a, b) or bool(torch.all((a == b) | (torch.isnan(a) & torch.isnan(b))))


def _inputs(B, Hq, Hkv, S, N, D, layout, device, seed):
    """Natural-order q, k, v on the CPU, and the GPU arguments of ra_ring."""
    q = rand((B, Hq, S, D), seed, torch.bfloat16)
    k = rand((B, Hkv, S, D), seed + 1, torch.bfloat16)
    v = rand((B, Hkv, S, D), seed + 2, torch.bfloat16)
    if device < 0:
        return q, k, v, [t.cuda() for t in (q, k, v)], np.arange(S)
    pos = OL.device_positions(S, N, layout, device)
    kd = torch.from_numpy(OL.to_device_order(k.float().numpy(), N, layout, axis=2)).bfloat16()
    vd = torch.from_numpy(OL.to_device_order(v.float().numpy(), N, layout, axis=2)).bfloat16()
    return q, k, v, [q[:, :, pos].contiguous().cuda(), kd.cuda(), vd.cuda()], pos


CASES = [  # (B, Hq, Hkv, S, N, D, layout, device)
    (1, 16, 4, 8192, 8, 128, "contiguous", -1),
    (1, 16, 4, 8192, 8, 128, "zigzag", -1),
    (1, 16, 4, 8192, 8, 128, "striped", -1),   # whole striped ring: items tile-major
    (1, 16, 4, 65536, 8, 128, "striped", 5),
    (1, 16, 4, 65536, 8, 128, "zigzag", 3),
    (2, 8, 2, 16384, 8, 64, "contiguous", -1),  # 4-wave kernel, two workgroups per CU
    (2, 8, 2, 16384, 8, 32, "zigzag", -1),
]


# one XCD nearly stalled: it gives away almost all of its list
STALL = [1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 0.05]


@pytest.mark.parametrize("case,speeds", [(c, SKEW) for c in CASES] + [(CASES[0], STALL)],
                         ids=lambda c: (f"B{c[0]}_D{c[5]}_{c[6]}_S{c[3]}_p{c[7]}"
                                        if isinstance(c, tuple) else
                                        ("stall" if c == STALL else "skew")))
def test_split_gives_identical_results(case, speeds):
    B, Hq, Hkv, S, N, D, layout, device = case
    log(f"xcd split {case} speeds {speeds}")
    q, k, v, (qd, kd, vd), pos = _inputs(B, Hq, Hkv, S, N, D, layout, device, 77)
    grid, M, keep, dbeg, dcnt = ra.ra_xcd_plan(qd, kd, N, layout, True, device, speeds)
    assert grid > 8 * M and sum(dcnt) > 0, "the skewed speeds must give a split launch"
    log(f"  plan: M {M}, keep {keep}, received {dcnt}")
    try:
        ra.ra_xcd_speeds([1.0] * 8, set=True)  # fixed split
        out0, lse0 = ra.ring_attention(qd, kd, vd, N, layout, True, device)
        ra.ra_xcd_speeds(speeds, set=True)
        out1, lse1 = ra.ring_attention(qd, kd, vd, N, layout, True, device)
        torch.cuda.synchronize()
    finally:
        ra.ra_xcd_speeds(None, set=True)
    assert _same(out0, out1) and _same(lse0, lse1), "results depend on the split"
    # oracle on sampled rows: the first and last rows and a seeded spread
    n = out1.shape[2]
    rows = np.unique(np.concatenate([[0, 1, n - 1], np.random.default_rng(5).integers(0, n, 40)]))
    ro, rl = O1.full_attention(q[:, :, pos[rows]], k, v, q_pos=pos[rows], k_pos=np.arange(S),
                               causal=True)
    check(out1[:, :, rows], lse1[:, :, rows], ro, rl, torch.bfloat16, f"{case} sampled rows")


def test_split_launch_in_a_graph():
    B, Hq, Hkv, S, N, D, layout = 1, 16, 4, 8192, 8, 128, "zigzag"
    log("xcd split in a graph")
    _, _, _, (q, k, v), _ = _inputs(B, Hq, Hkv, S, N, D, layout, -1, 91)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    try:
        ra.ra_xcd_speeds(SKEW, set=True)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            ra.ra_ring(q, k, v, out, lse, N, layout, True, -1, None, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ra.ra_ring(q, k, v, out, lse, N, layout, True, -1, None)
        ra.ra_xcd_speeds([1.0] * 8, set=True)
        for rep in range(3):
            q.mul_(-1.0 if rep % 2 else 1.0)
            g.replay()
            torch.cuda.synchronize()
            out_g, lse_g = out.clone(), lse.clone()
            out_e, lse_e = ra.ring_attention(q, k, v, N, layout, True)  # fixed split
            torch.cuda.synchronize()
            assert _same(out_g, out_e) and _same(lse_g, lse_e), f"replay {rep} differs"
    finally:
        ra.ra_xcd_speeds(None, set=True)


def test_speed_estimate_is_measured():
    # launches of about 8 ms: long enough to be measured (1 ms or more) and
    # with enough work items per CU for the split's model
    B, Hq, Hkv, S, N, D = 1, 32, 8, 32768, 8, 128
    log("xcd speed measurement")
    _, _, _, (q, k, v), _ = _inputs(B, Hq, Hkv, S, N, D, "contiguous", -1, 55)
    # the default mode measures nothing
    ra.ra_xcd_speeds(None, set=True)
    for _ in range(4):
        ra.ring_attention(q, k, v, N, "contiguous", True)
        torch.cuda.synchronize()
    speeds, nmeas = ra.ra_xcd_speeds()
    assert nmeas == 0 and speeds == [1.0] * 8
    try:
        ra.ra_xcd_speeds(measure=True)
        for _ in range(32):
            ra.ring_attention(q, k, v, N, "contiguous", True)
            torch.cuda.synchronize()
        speeds, nmeas = ra.ra_xcd_speeds()
    finally:
        ra.ra_xcd_speeds(None, set=True)
    log(f"  speeds {[round(x, 4) for x in speeds]} from {nmeas} measurements")
    assert nmeas >= 1
    assert abs(sum(speeds) / 8 - 1.0) < 1e-3
    assert all(0.75 <= x <= 1.33 for x in speeds)
