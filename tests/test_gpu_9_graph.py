"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on the
capturing stream) and replayed.  Every call only launches kernels on the
caller's stream (no allocation, no memset, no synchronisation), so a graph
holds exactly the kernels of an eager call.  Each graph is replayed several
times with eager work of the program and synchronisations in between, the
inputs are changed between replays, and every replay is compared bit for bit
with an eager call on the same inputs."""

import pytest
import torch

import blockwise_online_softmax_amd as ra
from gpu_helpers import log, rand

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _same(a, b):
    return torch.equal(a, b) or bool(torch.all((a == b) | (torch.isnan(a) & torch.isnan(b))))


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_ring_graph(layout):
    B, Hq, Hkv, S, N, D = 1, 4, 2, 1024, 4, 128
    log(f"graph ring {layout}")
    q = rand((B, Hq, S, D), 301, torch.bfloat16).cuda()
    k = rand((B, Hkv, S, D), 302, torch.bfloat16).cuda()
    v = rand((B, Hkv, S, D), 303, torch.bfloat16).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    nws = ra.ra_ring_workspace_bytes(q, k, N, layout, -1)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        ra.ra_ring(q, k, v, out, lse, N, layout, True, -1, ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ra.ra_ring(q, k, v, out, lse, N, layout, True, -1, ws)
    for rep in range(REPLAYS):
        # new inputs in place, then the graph, then an eager call to compare
        q.copy_(rand((B, Hq, S, D), 400 + rep, torch.bfloat16).cuda())
        v.mul_(-1.0 if rep % 2 else 1.0)
        g.replay()
        torch.cuda.synchronize()
        out_g, lse_g = out.clone(), lse.clone()
        out_e, lse_e = ra.ring_attention(q, k, v, N, layout, True)
        torch.cuda.synchronize()
        assert _same(out_g, out_e) and _same(lse_g, lse_e), f"replay {rep} differs"


def test_step_api_graph():
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 256, 192, 128
    log("graph step api")
    q = rand((B, Hq, Sq, D), 311, torch.bfloat16).cuda()
    ks = [rand((B, Hkv, Sk, D), 312 + j, torch.bfloat16).cuda() for j in range(3)]
    vs = [rand((B, Hkv, Sk, D), 322 + j, torch.bfloat16).cuda() for j in range(3)]
    qpos = torch.arange(Sq, dtype=torch.int32, device="cuda") + 3 * Sk - Sq
    kps = [torch.arange(Sk, dtype=torch.int32, device="cuda") + j * Sk for j in range(3)]
    st = ra.State(B, Hq, Sq, D)
    out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")

    def run(state, o, l_):
        ra.ra_state_init(state)
        for j in range(3):
            ra.ra_block_step(q, ks[j], vs[j], qpos, kps[j], ra.RA_MASK_CAUSAL, state)
        ra.ra_finalize(state, o, l_)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(st, out, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(st, out, lse)
    st2 = ra.State(B, Hq, Sq, D)
    for rep in range(REPLAYS):
        ks[rep % 3].copy_(rand((B, Hkv, Sk, D), 500 + rep, torch.bfloat16).cuda())
        g.replay()
        torch.cuda.synchronize()
        out_g, lse_g = out.clone(), lse.clone()
        m_g, l_g, acc_g = st.m.clone(), st.l.clone(), st.acc.clone()
        out_e = torch.empty_like(out)
        lse_e = torch.empty_like(lse)
        run(st2, out_e, lse_e)
        torch.cuda.synchronize()
        assert _same(out_g, out_e) and _same(lse_g, lse_e), f"replay {rep}: out / lse differ"
        assert _same(m_g, st2.m) and _same(l_g, st2.l) and _same(acc_g, st2.acc), \
            f"replay {rep}: state differs"


def test_merge_graph():
    rows, D = 4096, 128
    log("graph merge")
    g_ = torch.Generator(device="cpu").manual_seed(331)
    oa = torch.randn((rows, D), generator=g_).bfloat16().cuda()
    ob = torch.randn((rows, D), generator=g_).bfloat16().cuda()
    la = (torch.randn(rows, generator=g_) * 4).cuda()
    lb = (torch.randn(rows, generator=g_) * 4).cuda()
    out = torch.empty_like(oa)
    lse = torch.empty_like(la)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ra.ra_merge(oa, la, ob, lb, out, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ra.ra_merge(oa, la, ob, lb, out, lse)
    for rep in range(REPLAYS):
        la.add_(0.5)
        g.replay()
        torch.cuda.synchronize()
        out_g, lse_g = out.clone(), lse.clone()
        out_e, lse_e = torch.empty_like(out), torch.empty_like(lse)
        ra.ra_merge(oa, la, ob, lb, out_e, lse_e)
        torch.cuda.synchronize()
        assert _same(out_g, out_e) and _same(lse_g, lse_e), f"replay {rep} differs"
