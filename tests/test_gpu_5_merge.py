"""Merge of two partial results over disjoint key sets (ra_state_merge,
ra_merge) against the oracle's merge (oracle/merge.py) and full attention.

Keys are split into two sets by a seeded random partition (not a contiguous
cut), each set is folded into its own state with ra_block_step, and the two
are merged: as running states, or finalized first and merged as (out, lse).
The result must equal causal full attention over all keys (O1) to the usual
tolerances.  Each merge kernel is also checked on its own: its output against
oracle/merge.py applied to the very inputs it was given (the GPU's partial
states / partial outputs), where the only error left is fp32 arithmetic and,
for bf16, the rounding of the merged output.
"""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
from oracle import attention as O1
from oracle import merge as O3
from gpu_helpers import check, log, maxerr, rand, to_np

pytestmark = pytest.mark.gpu

CAUSAL = ra.RA_MASK_CAUSAL


def i32(a):
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


def half_state(q, k, v, qp, kp, sel):
    """State of q over the keys picked by `sel` (bool mask over key rows)."""
    B, Hq, Sq, D = q.shape
    st = ra.State(B, Hq, Sq, D)
    ra.ra_state_init(st)
    idx = np.nonzero(sel)[0]
    if len(idx):
        ra.ra_block_step(q, k[:, :, idx].contiguous(), v[:, :, idx].contiguous(), i32(qp),
                         i32(kp[idx]), CAUSAL, st)
    return st


def finalize(st, dtype):
    B, Hq, Sq, D = st.shape
    out = torch.empty((B, Hq, Sq, D), dtype=dtype, device="cuda")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    ra.ra_finalize(st, out, lse)
    return out, lse


def split(S, seed, frac=0.45):
    rng = np.random.default_rng(seed)
    sel = rng.random(S) < frac
    sel[0] = True    # the row at position 0 sees only side a
    sel[1] = False
    return sel


def check_state_merge_kernel(a, b, m, what):
    """GPU merged state vs oracle merge_states of the GPU's own halves."""
    ga = tuple(to_np(t) for t in (a.m, a.l, a.acc))
    gb = tuple(to_np(t) for t in (b.m, b.l, b.acc))
    rm, rl, racc = O3.merge_states(ga, gb)
    gm, gl, gacc = (to_np(t) for t in (m.m, m.l, m.acc))
    # the merged max is a max of fp32 values: exact
    assert np.array_equal(gm, rm), f"{what}: merged m differs"
    seen = rl > 0
    assert np.all(gl[~seen] == 0) and np.all(gacc[~seen] == 0), f"{what}: empty rows"
    el = float(np.max(np.abs(gl[seen] - rl[seen]) / rl[seen])) if seen.any() else 0.0
    eacc = float(np.max(np.abs(gacc[seen] - racc[seen]) / rl[seen][:, None])) if seen.any() else 0.0
    log(f"  {what}: state merge kernel rel l err {el:.2e}, acc err / l {eacc:.2e}")
    assert el <= 1e-6 and eacc <= 1e-5, f"{what}: l {el}, acc {eacc}"


def check_out_merge_kernel(oa, la, ob, lb, oo, lo, dtype, what):
    """GPU merged (out, lse) vs oracle merge_outputs of the GPU's own inputs."""
    ro, rl = O3.merge_outputs(to_np(oa), to_np(la), to_np(ob), to_np(lb))
    go, gl = to_np(oo), to_np(lo)
    # lse is rounded to fp32 once (half an ulp, <= 2^-24 of 2|lse|) after
    # fp32 arithmetic; allow 4x that plus a small absolute term
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{what}: empty rows differ"
    fin = np.isfinite(rl)
    el = np.abs(gl[fin] - rl[fin])
    bad_l = el > np.abs(rl[fin]) * 2.0 ** -22 + 1e-6
    # out: fp32 arithmetic leaves a few fp32 ulps of the larger term
    # (<= 2^-20 (|out_a| + |out_b|)); bf16 then rounds once to nearest (half
    # an ulp, <= 2^-8 of |out|)
    tol = np.abs(ro) * (2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -22) + \
        2.0 ** -20 * (np.abs(to_np(oa)) + np.abs(to_np(ob)))
    bad = np.abs(go - ro) > tol
    log(f"  {what}: out merge kernel max lse err {float(el.max(initial=0)):.2e}, "
        f"elements over bound: lse {int(bad_l.sum())}, out {int(bad.sum())}")
    assert not bad_l.any(), f"{what}: lse off by {float(el.max())}"
    assert not bad.any(), f"{what}: out off by {float(np.max(np.abs(go - ro)))}"


CASES = [
    # B, Hq, Hkv, S, D, dtype
    (1, 4, 2, 600, 128, torch.bfloat16),
    (2, 2, 1, 333, 64, torch.bfloat16),
    (1, 3, 3, 257, 32, torch.float32),
    (1, 2, 2, 100, 16, torch.float32),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,dtype", CASES)
def test_merge_equals_full_attention(B, Hq, Hkv, S, D, dtype):
    log(f"merge B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} {dtype}")
    q = rand((B, Hq, S, D), 501, dtype)
    k = rand((B, Hkv, S, D), 502, dtype)
    v = rand((B, Hkv, S, D), 503, dtype)
    pos = np.arange(S)
    ro, rl = O1.full_attention(q, k, v, causal=True)
    sel = split(S, 504)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    a = half_state(qg, kg, vg, pos, pos, sel)
    b = half_state(qg, kg, vg, pos, pos, ~sel)

    # running states merged, then finalized
    m = ra.State(B, Hq, S, D)
    ra.ra_state_merge(a, b, m)
    torch.cuda.synchronize()
    check_state_merge_kernel(a, b, m, "a+b")
    out, lse = finalize(m, dtype)
    torch.cuda.synchronize()
    check(out, lse, ro, rl, dtype, "state merge vs O1")

    # finalized halves merged as (out, lse)
    oa, la = finalize(a, dtype)
    ob, lb = finalize(b, dtype)
    oo = torch.empty_like(oa)
    lo = torch.empty_like(la)
    ra.ra_merge(oa, la, ob, lb, oo, lo)
    torch.cuda.synchronize()
    check_out_merge_kernel(oa, la, ob, lb, oo, lo, dtype, "a+b")
    check(oo, lo, ro, rl, dtype, "out merge vs O1")
    # row 0 sees key 0 only, which is on side a: side b's lse there is -inf
    assert torch.isneginf(lb[..., 0]).all() and torch.isfinite(la[..., 0]).all()

    # merge order does not matter: b + a gives the same bits
    m2 = ra.State(B, Hq, S, D)
    ra.ra_state_merge(b, a, m2)
    oo2, lo2 = torch.empty_like(oa), torch.empty_like(la)
    ra.ra_merge(ob, lb, oa, la, oo2, lo2)
    torch.cuda.synchronize()
    assert torch.equal(m2.acc, m.acc) and torch.equal(m2.l, m.l) and torch.equal(m2.m, m.m)
    assert torch.equal(oo2, oo) and torch.equal(lo2, lo)

    # in place: out is side a's or side b's buffers; same bits as out of place
    oa0, la0 = oa.clone(), la.clone()
    ra.ra_merge(oa, la, ob, lb, oa, la)
    ra.ra_merge(oa0, la0, ob, lb, ob, lb)
    ra.ra_state_merge(a, b, b)
    torch.cuda.synchronize()
    assert torch.equal(oa, oo) and torch.equal(la, lo)
    assert torch.equal(ob, oo) and torch.equal(lb, lo)
    assert torch.equal(b.acc, m.acc) and torch.equal(b.l, m.l) and torch.equal(b.m, m.m)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_merge_with_empty(dtype, D):
    """An empty side (no visible key) is an identity, bit for bit; two empty
    sides stay empty (m = -inf, l = 0, acc = 0; out = 0, lse = -inf)."""
    B, Hq, S = 1, 2, 192
    log(f"merge empty {dtype} D={D}")
    q = rand((B, Hq, S, D), 511, dtype).cuda()
    k = rand((B, Hq, S, D), 512, dtype).cuda()
    v = rand((B, Hq, S, D), 513, dtype).cuda()
    pos = np.arange(S)
    a = half_state(q, k, v, pos, pos, np.ones(S, dtype=bool))
    e = half_state(q, k, v, pos, pos, np.zeros(S, dtype=bool))
    for x, y in ((a, e), (e, a)):
        m = ra.State(B, Hq, S, D)
        ra.ra_state_merge(x, y, m)
        torch.cuda.synchronize()
        assert torch.equal(m.m, a.m) and torch.equal(m.l, a.l) and torch.equal(m.acc, a.acc)
    m = ra.State(B, Hq, S, D)
    ra.ra_state_merge(e, e, m)
    oa, la = finalize(a, dtype)
    oe, le = finalize(e, dtype)
    oo, lo = torch.empty_like(oa), torch.empty_like(la)
    ra.ra_merge(oe, le, oa, la, oo, lo)
    torch.cuda.synchronize()
    assert torch.isneginf(m.m).all() and (m.l == 0).all() and (m.acc == 0).all()
    assert torch.equal(oo, oa) and torch.equal(lo, la)
    ra.ra_merge(oe, le, oe, le, oo, lo)
    torch.cuda.synchronize()
    assert (oo == 0).all() and torch.isneginf(lo).all()


def test_merge_full_size_bf16():
    """A 32K-token bf16 share: two 4096-row query blocks x 32 heads x D 128
    per side (1M rows), with lse drawn over a wide range so that either side
    dominates or they tie; checked against the oracle merge on every row."""
    rows_shape = (1, 32, 32768)
    D = 128
    log("merge full size bf16 1x32x32768x128")
    g = torch.Generator(device="cpu")
    g.manual_seed(521)
    oa = torch.randn(rows_shape + (D,), generator=g).bfloat16()
    ob = torch.randn(rows_shape + (D,), generator=g).bfloat16()
    la = torch.randn(rows_shape, generator=g) * 20
    lb = torch.randn(rows_shape, generator=g) * 20
    lb[..., ::7] = la[..., ::7]                  # ties
    la[..., 3::11] = -float("inf")               # side a empty on some rows
    lb[..., 5::13] = -float("inf")               # side b empty on others (some both)
    oa[la.isneginf()] = 0
    ob[lb.isneginf()] = 0
    ga, gb, gla, glb = (t.cuda() for t in (oa, ob, la, lb))
    oo, lo = torch.empty_like(ga), torch.empty_like(gla)
    ra.ra_merge(ga, gla, gb, glb, oo, lo)
    torch.cuda.synchronize()
    check_out_merge_kernel(oa, la, ob, lb, oo, lo, torch.bfloat16, "1M rows")
