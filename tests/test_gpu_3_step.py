"""The composable state API (ra_state_init / ra_block_step / ra_finalize)
against the oracle's recurrence and full attention."""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
from oracle import attention as O1
from oracle import layouts as OL
from oracle import ring as O2
from gpu_helpers import TOL, check, log, maxerr, rand, to_np

pytestmark = pytest.mark.gpu

CAUSAL = ra.RA_MASK_CAUSAL


def i32(a):
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


def new_state(B, Hq, Sq, D):
    st = ra.State(B, Hq, Sq, D)
    ra.ra_state_init(st)
    return st


def check_state(st, ostates, dtype, what):
    """GPU state vs the oracle's (m, l, o) per (b, h): m, partial out o/l and m + ln l."""
    m = to_np(st.m)
    l_ = to_np(st.l)
    acc = to_np(st.acc)
    tol_o, tol_l = TOL[dtype]
    for (b, h), (om, ol, oo) in ostates.items():
        seen = ol > 0
        assert np.array_equal(np.isinf(m[b, h]), ~seen), f"{what}: empty rows differ"
        em = maxerr(m[b, h][seen], om[seen])
        assert em <= 1e-4, f"{what}: m error {em}"
        gpart = acc[b, h][seen] / l_[b, h][seen][:, None]
        opart = oo[seen] / ol[seen][:, None]
        eo = maxerr(gpart, opart)
        el = maxerr(m[b, h][seen] + np.log(l_[b, h][seen]), om[seen] + np.log(ol[seen]))
        assert eo <= tol_o and el <= tol_l, f"{what}: partial out {eo}, partial lse {el}"
        assert np.all(acc[b, h][~seen] == 0) and np.all(l_[b, h][~seen] == 0)


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 32), (torch.bfloat16, 16)])
def test_ring_by_steps(layout, dtype, D):
    """Each device folds the N blocks in ring order, one ra_block_step each;
    the state after every step matches the oracle recurrence and the
    finalized output matches full attention."""
    B, Hq, Hkv, S, N = 1, 4, 2, 1024, 4
    log(f"steps {layout} {dtype} D={D}")
    q = rand((B, Hq, S, D), 61, dtype)
    k = rand((B, Hkv, S, D), 62, dtype)
    v = rand((B, Hkv, S, D), 63, dtype)
    ro, rl = O1.full_attention(q, k, v, causal=True)
    qf, kf, vf = (t.double().numpy() for t in (q, k, v))
    scale = 1.0 / np.sqrt(D)
    G = Hq // Hkv
    for p in (0, N - 1):
        qp = OL.device_positions(S, N, layout, p)
        Qp = q[:, :, qp].contiguous().cuda()
        st = new_state(B, Hq, len(qp), D)
        ost = {(0, h): O2.init_state(len(qp), D) for h in range(Hq)}
        for s in range(N):
            j = (p - s) % N
            kp = OL.device_positions(S, N, layout, j)
            ra.ra_block_step(Qp, k[:, :, kp].contiguous().cuda(), v[:, :, kp].contiguous().cuda(),
                             i32(qp), i32(kp), CAUSAL, st)
            vis = kp[None, :] <= qp[:, None]
            for h in range(Hq):
                ost[(0, h)] = O2.absorb_block(ost[(0, h)], qf[0, h][qp], kf[0, h // G][kp],
                                              vf[0, h // G][kp], scale, vis)
            torch.cuda.synchronize()
            check_state(st, ost, dtype, f"p={p} step {s}")
        out = torch.empty((B, Hq, len(qp), D), dtype=dtype, device="cuda")
        lse = torch.empty((B, Hq, len(qp)), dtype=torch.float32, device="cuda")
        ra.ra_finalize(st, out, lse)
        check(out, lse, ro[:, :, qp], rl[:, :, qp], dtype, f"steps p={p} {layout}")


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_order_invariance_and_resume(dtype, D):
    """Blocks folded in a shuffled order give the same result; a state copied
    out mid-ring and resumed in fresh buffers gives bit-identical output."""
    B, Hq, Hkv, S, N = 1, 4, 1, 1536, 6
    q = rand((B, Hq, S, D), 71, dtype)
    k = rand((B, Hkv, S, D), 72, dtype)
    v = rand((B, Hkv, S, D), 73, dtype)
    ro, rl = O1.full_attention(q, k, v, causal=True)
    layout = "striped"
    p = 2
    qp = OL.device_positions(S, N, layout, p)
    Qp = q[:, :, qp].contiguous().cuda()
    blocks = {}
    for j in range(N):
        kp = OL.device_positions(S, N, layout, j)
        blocks[j] = (k[:, :, kp].contiguous().cuda(), v[:, :, kp].contiguous().cuda(), i32(kp))
    rng = np.random.default_rng(5)
    results = []
    for order in ([(p - s) % N for s in range(N)], list(rng.permutation(N))):
        st = new_state(B, Hq, len(qp), D)
        for j in order:
            ra.ra_block_step(Qp, blocks[j][0], blocks[j][1], i32(qp), blocks[j][2], CAUSAL, st)
        out = torch.empty((B, Hq, len(qp), D), dtype=dtype, device="cuda")
        lse = torch.empty((B, Hq, len(qp)), dtype=torch.float32, device="cuda")
        ra.ra_finalize(st, out, lse)
        check(out, lse, ro[:, :, qp], rl[:, :, qp], dtype, f"order {order}")
        results.append((out, lse))
    # resume: 3 steps, copy the state to new buffers, 3 more steps
    order = [(p - s) % N for s in range(N)]
    st = new_state(B, Hq, len(qp), D)
    for j in order[:3]:
        ra.ra_block_step(Qp, blocks[j][0], blocks[j][1], i32(qp), blocks[j][2], CAUSAL, st)
    st2 = ra.State(B, Hq, len(qp), D)
    st2.m.copy_(st.m)
    st2.l.copy_(st.l)
    st2.acc.copy_(st.acc)
    del st
    for j in order[3:]:
        ra.ra_block_step(Qp, blocks[j][0], blocks[j][1], i32(qp), blocks[j][2], CAUSAL, st2)
    out = torch.empty((B, Hq, len(qp), D), dtype=dtype, device="cuda")
    lse = torch.empty((B, Hq, len(qp)), dtype=torch.float32, device="cuda")
    ra.ra_finalize(st2, out, lse)
    assert torch.equal(out, results[0][0]) and torch.equal(lse, results[0][1])


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 8)])
def test_arbitrary_positions_and_ragged(dtype, D):
    """Unsorted positions, ragged sizes, a row that sees nothing, Sk = 1."""
    rng = np.random.default_rng(81)
    for (Sq, Sk) in [(77, 130), (200, 1), (1, 65), (300, 257)]:
        B, Hq, Hkv = 2, 4, 2
        q = rand((B, Hq, Sq, D), 82 + Sq, dtype)
        k = rand((B, Hkv, Sk, D), 83 + Sk, dtype)
        v = rand((B, Hkv, Sk, D), 84 + Sk, dtype)
        qpos = rng.permutation(np.arange(Sq) * 3 + 5)
        kpos = rng.permutation(np.arange(Sk) * 2 + 4)
        qpos[0] = -1  # sees no key
        for mask in (ra.RA_MASK_NONE, CAUSAL):
            st = new_state(B, Hq, Sq, D)
            ra.ra_block_step(q.cuda(), k.cuda(), v.cuda(), i32(qpos), i32(kpos), mask, st)
            out = torch.empty((B, Hq, Sq, D), dtype=dtype, device="cuda")
            lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
            ra.ra_finalize(st, out, lse)
            ro, rl = O1.full_attention(q, k, v, q_pos=qpos, k_pos=kpos, causal=(mask == CAUSAL))
            check(out, lse, ro, rl, dtype, f"Sq={Sq} Sk={Sk} mask={mask}")
            if mask == CAUSAL:
                assert torch.all(out[:, :, 0] == 0) and torch.all(torch.isneginf(lse[:, :, 0]))


def test_finalize_fp32_output_from_bf16_state():
    B, Hq, Hkv, S, D = 1, 2, 1, 256, 128
    q = rand((B, Hq, S, D), 91, torch.bfloat16)
    k = rand((B, Hkv, S, D), 92, torch.bfloat16)
    v = rand((B, Hkv, S, D), 93, torch.bfloat16)
    st = new_state(B, Hq, S, D)
    pos = i32(np.arange(S))
    ra.ra_block_step(q.cuda(), k.cuda(), v.cuda(), pos, pos, CAUSAL, st)
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    ra.ra_finalize(st, out, lse)
    ro, rl = O1.full_attention(q, k, v, causal=True)
    check(out, lse, ro, rl, torch.bfloat16, "fp32 out from bf16 inputs")


def test_empty_state_finalize():
    st = new_state(1, 2, 10, 32)
    out = torch.full((1, 2, 10, 32), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.zeros((1, 2, 10), dtype=torch.float32, device="cuda")
    ra.ra_finalize(st, out, lse)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(torch.isneginf(st.m)) and torch.all(st.l == 0) and torch.all(st.acc == 0)
