"""The C ABI on the host, no GPU: libra.so loads, exports every function
include/ra.h declares, and every invalid-argument path returns its status and
a message before anything is launched (validation never touches the device,
so fake but aligned device addresses are safe here)."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

from blockwise_online_softmax_amd import capi
from blockwise_online_softmax_amd.capi import RaDims, RaState

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")

FAKE = 0x7F0000000000  # aligned, never dereferenced: validation rejects first


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(capi.LIB_PATH):
        pytest.fail("libra.so not built: run python -m blockwise_online_softmax_amd.build")
    return capi.load()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(capi.EXPORTED), names
    dyn = subprocess.run(["nm", "-D", "--defined-only", capi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ra_[a-z_]+)\b", dyn))
    for n in names:
        assert n in exported, f"{n} not exported"
        assert getattr(lib, n) is not None
    assert lib.ra_version() == 105


def dims(B=1, Hq=4, Hkv=2, Sq=128, Sk=128, D=128, dtype=1, scale=0.0):
    return RaDims(B, Hq, Hkv, Sq, Sk, D, dtype, scale)


def state(B=1, Hq=4, Sq=128, D=128, m=FAKE, l=FAKE + 4096, acc=FAKE + 8192):
    return RaState(m, l, acc, B, Hq, Sq, D)


def expect(status, code, fragment):
    assert status == code, (capi.STATUS_NAMES.get(status), capi.last_error())
    assert fragment.lower() in capi.last_error().lower(), capi.last_error()


def step(lib, d, st, mask=0, q=FAKE, k=FAKE, v=FAKE, qp=FAKE, kp=FAKE):
    return lib.ra_block_step(q, k, v, qp, kp, mask, ctypes.byref(d) if d is not None else None,
                             ctypes.byref(st) if st is not None else None, None)


def test_state_init_errors(lib):
    expect(lib.ra_state_init(None, None), capi.RA_ERR_NULL, "state")
    expect(lib.ra_state_init(ctypes.byref(state(m=0)), None), capi.RA_ERR_NULL, "non-NULL")
    expect(lib.ra_state_init(ctypes.byref(state(D=100)), None), capi.RA_ERR_UNSUPPORTED, "head dim")
    expect(lib.ra_state_init(ctypes.byref(state(Sq=0)), None), capi.RA_ERR_SHAPE, "range")
    expect(lib.ra_state_init(ctypes.byref(state(acc=FAKE + 8)), None), capi.RA_ERR_SHAPE, "align")


def test_block_step_errors(lib):
    st = state()
    expect(step(lib, None, st), capi.RA_ERR_NULL, "dims")
    expect(step(lib, dims(dtype=5), st), capi.RA_ERR_DTYPE, "dtype")
    expect(step(lib, dims(Hq=3), state(Hq=3)), capi.RA_ERR_SHAPE, "multiple")
    expect(step(lib, dims(D=48), state(D=48)), capi.RA_ERR_UNSUPPORTED, "head dim")
    expect(step(lib, dims(), st, mask=3), capi.RA_ERR_ENUM, "mask")
    expect(step(lib, dims(), st, mask=1, qp=None), capi.RA_ERR_NULL, "q_pos")
    expect(step(lib, dims(), st, q=None), capi.RA_ERR_NULL, "non-NULL")
    expect(step(lib, dims(Sq=64), st), capi.RA_ERR_SHAPE, "does not match")
    expect(step(lib, dims(), st, q=FAKE + 2), capi.RA_ERR_SHAPE, "aligned")
    expect(step(lib, dims(Sk=0), st), capi.RA_ERR_SHAPE, ">= 1")
    expect(step(lib, dims(scale=float("nan")), st), capi.RA_ERR_SHAPE, "finite")
    expect(step(lib, dims(Sq=1 << 31), state(Sq=1 << 31)), capi.RA_ERR_SHAPE, "2^31")


def test_finalize_errors(lib):
    st = state()
    expect(lib.ra_finalize(ctypes.byref(st), None, None, 1, None), capi.RA_ERR_NULL, "out")
    expect(lib.ra_finalize(ctypes.byref(st), FAKE, None, 9, None), capi.RA_ERR_DTYPE, "dtype")
    expect(lib.ra_finalize(None, FAKE, None, 1, None), capi.RA_ERR_NULL, "state")
    expect(lib.ra_finalize(ctypes.byref(st), FAKE + 2, None, 1, None), capi.RA_ERR_SHAPE, "align")


def ring(lib, d, N=8, layout=0, causal=1, device=-1, ws=None, wsb=0, out=FAKE, lse=FAKE):
    return lib.ra_ring(FAKE, FAKE, FAKE, out, lse, ctypes.byref(d), N, layout, causal, device,
                       ws, wsb, None)


def test_ring_errors(lib):
    expect(ring(lib, dims(), N=0), capi.RA_ERR_SHAPE, "N must")
    expect(ring(lib, dims(), layout=7), capi.RA_ERR_ENUM, "layout")
    expect(ring(lib, dims(), device=8), capi.RA_ERR_ENUM, "device")
    expect(ring(lib, dims(), device=-2), capi.RA_ERR_ENUM, "device")
    expect(ring(lib, dims(Sq=120, Sk=120), N=16), capi.RA_ERR_SHAPE, "divisible")
    expect(ring(lib, dims(Sq=120, Sk=120), N=8, layout=2), capi.RA_ERR_SHAPE, "zigzag")
    expect(ring(lib, dims(Sq=64), N=8), capi.RA_ERR_SHAPE, "Sq == Sk")
    expect(ring(lib, dims(Sq=128), N=8, device=3), capi.RA_ERR_SHAPE, "S/N")
    expect(ring(lib, dims(), causal=2), capi.RA_ERR_ENUM, "causal")
    expect(ring(lib, dims(), out=None), capi.RA_ERR_NULL, "non-NULL")
    # fp32 inputs run on device-ordered copies in the workspace
    f32 = dims(dtype=0)
    need = lib.ra_ring_workspace_bytes(ctypes.byref(f32), 8, 1, -1)
    assert 0 < need < (1 << 40)
    expect(ring(lib, f32, layout=1), capi.RA_ERR_WORKSPACE, "required")
    expect(ring(lib, f32, layout=1, ws=FAKE, wsb=need - 1), capi.RA_ERR_WORKSPACE, "small")
    expect(ring(lib, f32, layout=2, ws=FAKE + 16, wsb=need), capi.RA_ERR_WORKSPACE, "256")


def test_workspace_bytes(lib):
    def ws(d, N, layout, device):
        return lib.ra_ring_workspace_bytes(ctypes.byref(d), N, layout, device)

    bad = ctypes.c_size_t(-1).value
    assert ws(dims(Hq=3), 8, 0, -1) == bad and "multiple" in capi.last_error()
    assert ws(dims(), 8, 0, -1) == 0 and capi.last_error() == ""
    assert ws(dims(Sq=16), 8, 2, 0) == 0  # a device share needs no workspace
    # bf16 with a matrix-core head dim: striped and zigzag whole rings are read
    # and written in natural order, no workspace
    d = dims(Hq=32, Hkv=8, Sq=65536, Sk=65536)
    for D in (32, 64, 128):
        assert ws(dims(Hq=32, Hkv=8, Sq=65536, Sk=65536, D=D), 8, 1, -1) == 0
        assert ws(dims(Hq=32, Hkv=8, Sq=65536, Sk=65536, D=D), 8, 2, -1) == 0
    # ... as long as a key/value head stays under 4 GiB (32-bit offsets from the
    # head's start); a larger one is permuted into the workspace
    S = 1 << 24  # 2^24 tokens x 128 x 2 bytes = 4 GiB per head
    assert ws(dims(Hq=1, Hkv=1, Sq=S - 16, Sk=S - 16), 8, 1, -1) == 0
    big = ws(dims(Hq=1, Hkv=1, Sq=S, Sk=S), 8, 1, -1)
    assert big == 4 * (S * 128 * 2) + S * 4 and capi.last_error() == ""
    # the vector kernels (fp32, or bf16 with D 8 / 16) work on device-ordered
    # copies: Q + out copies, K + V copies, lse copy
    for dtype, D, es in ((0, 128, 4), (1, 16, 2), (1, 8, 2)):
        d = dims(Hq=32, Hkv=8, Sq=65536, Sk=65536, D=D, dtype=dtype)
        q = 32 * 65536 * D * es
        kv = 8 * 65536 * D * es
        assert ws(d, 8, 1, -1) == 2 * q + 2 * kv + 32 * 65536 * 4


def test_merge_errors(lib):
    M = lib.ra_state_merge
    a, b = state(), state(m=FAKE + (1 << 20), l=FAKE + (1 << 20) + 4096, acc=FAKE + (2 << 20))
    r = ctypes.byref
    expect(M(None, r(b), r(a), None), capi.RA_ERR_NULL, "state")
    expect(M(r(a), r(b), r(state(Sq=64)), None), capi.RA_ERR_SHAPE, "equal")
    expect(M(r(a), r(state(D=64)), r(a), None), capi.RA_ERR_SHAPE, "equal")
    expect(M(r(a), r(b), r(state(D=100)), None), capi.RA_ERR_UNSUPPORTED, "head dim")
    # out.m on a.l's buffer, out.acc straddling b.acc, out.l == out.m
    expect(M(r(a), r(b), r(state(m=FAKE + 4096, l=FAKE + (3 << 20), acc=FAKE + (4 << 20))), None),
           capi.RA_ERR_SHAPE, "overlap")
    expect(M(r(a), r(b), r(state(m=FAKE + (3 << 20), l=FAKE + (3 << 20) + 4096,
                                 acc=FAKE + (2 << 20) + 256)), None), capi.RA_ERR_SHAPE, "overlap")
    expect(M(r(a), r(b), r(state(m=FAKE + (3 << 20), l=FAKE + (3 << 20), acc=FAKE + (4 << 20))), None),
           capi.RA_ERR_SHAPE, "overlap")

    G = lib.ra_merge
    oa, la, ob, lb, oo, lo = (FAKE + (i << 20) for i in range(6))

    def g(*args, rows=64, D=128, dtype=1):
        x = dict(zip(("oa", "la", "ob", "lb", "oo", "lo"), (oa, la, ob, lb, oo, lo)))
        x.update(dict(args))
        return G(x["oa"], x["la"], x["ob"], x["lb"], x["oo"], x["lo"], rows, D, dtype, None)

    expect(g(("lb", None)), capi.RA_ERR_NULL, "non-NULL")
    expect(g(dtype=4), capi.RA_ERR_DTYPE, "dtype")
    expect(g(rows=0), capi.RA_ERR_SHAPE, "rows")
    expect(g(D=96), capi.RA_ERR_UNSUPPORTED, "head dim")
    expect(g(("oo", oo + 4)), capi.RA_ERR_SHAPE, "misaligned")
    expect(g(("lo", la + 4)), capi.RA_ERR_SHAPE, "overlap")
    expect(g(("oo", lb)), capi.RA_ERR_SHAPE, "overlap")
    expect(g(("oo", ob + 64)), capi.RA_ERR_SHAPE, "overlap")


def test_vocab_ce_errors(lib):
    S = lib.ra_vocab_ce_shard
    L, T = FAKE, FAKE + (1 << 20)
    outs = (FAKE + (2 << 20), FAKE + (3 << 20), FAKE + (4 << 20))
    expect(S(None, 16, T, 4, 16, 0, 1, *outs, None), capi.RA_ERR_NULL, "logits")
    expect(S(L, 16, T, 4, 16, 0, 7, *outs, None), capi.RA_ERR_DTYPE, "dtype")
    expect(S(L, 16, T, 0, 16, 0, 1, *outs, None), capi.RA_ERR_SHAPE, "N must")
    expect(S(L, 8, T, 4, 16, 0, 1, *outs, None), capi.RA_ERR_SHAPE, "ld")
    expect(S(L + 1, 16, T, 4, 16, 0, 1, *outs, None), capi.RA_ERR_SHAPE, "misaligned")
    expect(S(L, 16, T + 4, 4, 16, 0, 1, *outs, None), capi.RA_ERR_SHAPE, "misaligned")
    expect(S(L, 16, T, 4, 16, 0, 1, None, outs[1], outs[2], None), capi.RA_ERR_NULL, "z_sum")
    expect(S(L, 16, T, 4, 16, 0, 1, outs[0], outs[0] + 8, outs[2], None), capi.RA_ERR_SHAPE, "overlap")
    expect(S(L, 16, T, 4, 16, 0, 1, L + 64, outs[1], outs[2], None), capi.RA_ERR_SHAPE, "overlap")
    C = lib.ra_vocab_ce_combine
    expect(C(*outs, 2, 4, outs[1] + 4, None, None), capi.RA_ERR_SHAPE, "overlap")
    expect(C(*outs, 2, 4, FAKE, FAKE + 8, None), capi.RA_ERR_SHAPE, "overlap")
    expect(C(*outs, 0, 4, FAKE, None, None), capi.RA_ERR_SHAPE, "t must")
    expect(C(*outs, 2, 4, None, None, None), capi.RA_ERR_NULL, "loss")
    G = lib.ra_vocab_ce_grad
    lse, grad = FAKE + (5 << 20), FAKE + (6 << 20)
    expect(G(L, 16, T, None, 4, 16, 0, 1.0, 1, grad, 16, None), capi.RA_ERR_NULL, "lse")
    expect(G(L, 16, T, lse, 4, 16, 0, float("inf"), 1, grad, 16, None), capi.RA_ERR_SHAPE, "finite")
    expect(G(L, 16, T, lse, 4, 16, 0, 1.0, 1, L + 32, 16, None), capi.RA_ERR_SHAPE, "overlap")
    expect(G(L, 16, T, lse, 4, 16, 0, 1.0, 1, grad, 8, None), capi.RA_ERR_SHAPE, "ldg")
    W = lib.ra_vocab_ce_workspace_bytes
    assert W(8192, 8) == 256 * ((3 * 8 * 8192 * 4 + 255) // 256) + 256 * ((128 * 4 + 255) // 256)
    assert W(0, 8) == ctypes.c_size_t(-1).value and "N must" in capi.last_error()
    need = W(4, 2)
    V = lib.ra_vocab_ce
    ws = FAKE + (8 << 20)
    expect(V(L, T, 4, 15, 2, 1, FAKE, FAKE, None, ws, need, None), capi.RA_ERR_SHAPE, "multiple")
    expect(V(L, T, 4, 16, 0, 1, FAKE, FAKE, None, ws, need, None), capi.RA_ERR_SHAPE, "t must")
    expect(V(L, T, 4, 16, 2, 1, FAKE, FAKE, None, None, 0, None), capi.RA_ERR_WORKSPACE, "required")
    expect(V(L, T, 4, 16, 2, 1, FAKE, FAKE, None, ws, need - 4, None), capi.RA_ERR_WORKSPACE, "small")
    expect(V(L, T, 4, 16, 2, 1, FAKE, FAKE, None, ws + 16, need, None), capi.RA_ERR_WORKSPACE, "256")
    expect(V(L, T, 4, 16, 2, 1, FAKE, None, None, ws, need, None), capi.RA_ERR_NULL, "mean_loss")
    expect(V(L, T, 4, 16, 2, 1, FAKE, ws + 64, None, ws, need, None), capi.RA_ERR_SHAPE, "overlap")
    expect(V(L, T, 4, 16, 2, 1, L, FAKE + (9 << 20), None, ws, need, None), capi.RA_ERR_SHAPE, "overlap")
    expect(G(L, 16, T, lse, 4, 16, 0, 1.0, 1, lse - 16, 16, None), capi.RA_ERR_SHAPE, "overlap")


def test_vocab_ce_static_errors(lib):
    """ra_vocab_ce_static validates like ra_vocab_ce and rejects sizes whose
    scratch exceeds its 8 MiB static array, all before any HIP call."""
    V = lib.ra_vocab_ce_static
    L, T = FAKE, FAKE + (1 << 30)
    loss, mean = FAKE + (2 << 30), FAKE + (3 << 30)
    W = lib.ra_vocab_ce_workspace_bytes
    assert W(87000, 8) <= 8 << 20 < W(100000, 8)
    expect(V(L, T, 100000, 16, 8, 1, loss, mean, None, None), capi.RA_ERR_WORKSPACE,
           "static scratch")
    expect(V(L, T, 4, 15, 2, 1, loss, mean, None, None), capi.RA_ERR_SHAPE, "multiple")
    expect(V(L, T, 4, 16, 0, 1, loss, mean, None, None), capi.RA_ERR_SHAPE, "t must")
    expect(V(None, T, 4, 16, 2, 1, loss, mean, None, None), capi.RA_ERR_NULL, "logits")
    expect(V(L, T, 4, 16, 2, 1, loss, None, None, None), capi.RA_ERR_NULL, "mean_loss")
    expect(V(L, T, 4, 16, 2, 1, L + 32, mean, None, None), capi.RA_ERR_SHAPE, "overlap")
    expect(V(L, T, 4, 16, 2, 1, loss, loss + 8, None, None), capi.RA_ERR_SHAPE, "overlap")
    if torch.cuda.device_count() == 0:  # valid arguments, but no device to run on
        expect(V(L, T, 4, 16, 2, 1, loss, mean, None, None), capi.RA_ERR_HIP, "device")


def test_layout_position_matches_oracle(lib):
    """The layout map the kernels use (compiled for the host through the ABI)
    against the oracle's maps, for every layout, whole sequences and device
    blocks, including N = 1 and odd block counts."""
    import numpy as np

    from oracle import layouts as OL

    for S, N in ((48, 4), (96, 8), (30, 3), (16, 1), (1024, 8), (64, 2)):
        for layout in ("contiguous", "striped", "zigzag"):
            if layout == "zigzag" and S % (2 * N):
                assert lib.ra_layout_position(S, N, capi.LAYOUT_IDS[layout], -1, 0) == -1
                assert "zigzag" in capi.last_error()
                continue
            whole = np.concatenate([OL.device_positions(S, N, layout, p) for p in range(N)])
            got = [lib.ra_layout_position(S, N, capi.LAYOUT_IDS[layout], -1, i) for i in range(S)]
            assert np.array_equal(np.array(got), whole), (S, N, layout)
            for p in (0, N - 1):
                want = OL.device_positions(S, N, layout, p)
                got = [lib.ra_layout_position(S, N, capi.LAYOUT_IDS[layout], p, i)
                       for i in range(S // N)]
                assert np.array_equal(np.array(got), want), (S, N, layout, p)
    assert lib.ra_layout_position(48, 4, 0, -1, 48) == -1 and "range" in capi.last_error()
    assert lib.ra_layout_position(48, 4, 0, 4, 0) == -1 and "device" in capi.last_error()
    assert lib.ra_layout_position(48, 4, 9, -1, 0) == -1 and "layout" in capi.last_error()
    assert lib.ra_layout_position(48, 5, 0, -1, 0) == -1 and "divisible" in capi.last_error()


def test_permute_and_positions_errors(lib):
    P = lib.ra_permute
    expect(P(None, FAKE, 1, 16, 256, 4, 0, 0, None), capi.RA_ERR_NULL, "src")
    expect(P(FAKE, FAKE, 1, 16, 6, 4, 0, 0, None), capi.RA_ERR_SHAPE, "multiple of 4")
    expect(P(FAKE, FAKE, 1, 16, 256, 4, 5, 0, None), capi.RA_ERR_ENUM, "layout")
    expect(P(FAKE, FAKE, 1, 16, 256, 4, 1, 2, None), capi.RA_ERR_ENUM, "inverse")
    expect(P(FAKE, FAKE, 1, 18, 256, 4, 1, 0, None), capi.RA_ERR_SHAPE, "divisible")
    expect(P(FAKE, FAKE, 1, 12, 256, 4, 2, 0, None), capi.RA_ERR_SHAPE, "zigzag")
    expect(P(FAKE + 4, FAKE, 1, 16, 256, 4, 1, 0, None), capi.RA_ERR_SHAPE, "misaligned")
    Q = lib.ra_positions
    expect(Q(None, 16, 4, 0, -1, None), capi.RA_ERR_NULL, "pos")
    expect(Q(FAKE, 16, 4, 0, 4, None), capi.RA_ERR_ENUM, "device")
    expect(Q(FAKE, 16, 4, 9, 0, None), capi.RA_ERR_ENUM, "layout")
    expect(Q(FAKE, 15, 4, 0, 0, None), capi.RA_ERR_SHAPE, "divisible")


def test_python_binding_rejects_cpu_tensors():
    import torch

    x = torch.zeros(1, 1, 8, 8)
    with pytest.raises(ValueError, match="GPU"):
        capi.ra_ring(x, x, x, x, torch.zeros(1, 1, 8), 1)


# ---- work split over the XCDs (host planner) ----

def _xcd_item(M, keep, dbeg, dcnt, w):
    """Item of workgroup w under a plan, as include/ra.h describes the split."""
    x, sl = w % 8, w // 8
    if sl < dcnt[x]:  # donated items first
        idx, y = dbeg[x] + sl, 0
        while y < 7 and idx >= M - keep[y]:
            idx -= M - keep[y]
            y += 1
        return y * M + idx
    own = sl - dcnt[x]
    return x * M + (M - keep[x]) + own if own < keep[x] else -1


def _plan(B, Hq, Hkv, S, D, N, layout, causal, device=-1, speeds=None, dtype=torch.bfloat16):
    Sq = S if device < 0 else S // N
    q = torch.empty((B, Hq, Sq, D), dtype=dtype, device="meta")
    k = torch.empty((B, Hkv, S, D), dtype=dtype, device="meta")
    return capi.ra_xcd_plan(q, k, N, layout, causal, device, speeds)


SKEW = [1.0, 0.97, 1.02, 0.96, 1.06, 0.99, 1.0, 0.95]


@pytest.mark.parametrize("layout,causal,device", [
    ("contiguous", True, -1), ("zigzag", True, -1), ("striped", True, -1),
    ("contiguous", False, -1), ("zigzag", True, 0), ("zigzag", True, 5)])
def test_xcd_plan_is_a_bijection(layout, causal, device):
    S = 32768 if device < 0 else 262144
    W = 32 * (S // 256) if device < 0 else 32 * (S // 8 // 256)
    grid, M, keep, dbeg, dcnt = _plan(1, 32, 8, S, 128, 8, layout, causal, device, SKEW)
    assert M * 8 == W and grid % 8 == 0
    assert grid == 8 * max(k + c for k, c in zip(keep, dcnt))
    items = [_xcd_item(M, keep, dbeg, dcnt, w) for w in range(grid)]
    got = sorted(i for i in items if i >= 0)
    assert got == list(range(W))
    # an XCD's own items (the last keep[x] of its longest-first list, so its
    # shortest) follow the ones it receives; an XCD that gives items away
    # receives none
    for x in range(8):
        own = [items[(dcnt[x] + s) * 8 + x] for s in range(keep[x])]
        assert own == [x * M + (M - keep[x]) + s for s in range(keep[x])]
        assert keep[x] == M or dcnt[x] == 0


@pytest.mark.parametrize("speeds", [
    [1, 1, 1, 1, 1, 1, 1, 0.05],          # one XCD nearly stalled: it may keep nothing
    [10, 1, 1, 1, 1, 1, 1, 1],            # one XCD far faster than the rest
    [1, 2, 1, 2, 1, 2, 1, 2]])
def test_xcd_plan_extreme_speeds_stay_a_bijection(speeds):
    """Speeds far outside the measured range still give a plan that maps the
    grid one-to-one onto the items (or the fixed split)."""
    S, W = 32768, 32 * (32768 // 256)
    grid, M, keep, dbeg, dcnt = _plan(1, 32, 8, S, 128, 8, "contiguous", True, -1, speeds)
    assert M * 8 == W and grid % 8 == 0
    items = [_xcd_item(M, keep, dbeg, dcnt, w) for w in range(grid)]
    assert sorted(i for i in items if i >= 0) == list(range(W))
    slow = min(range(8), key=lambda x: speeds[x])
    assert keep[slow] < M  # the slowest XCD gives work away


def test_xcd_plan_equal_speeds_is_the_fixed_split():
    grid, M, keep, dbeg, dcnt = _plan(1, 32, 8, 32768, 128, 8, "contiguous", True)
    assert (grid, M) == (4096, 512)
    assert keep == [512] * 8 and dcnt == [0] * 8


def test_xcd_plan_moves_work_from_slow_to_fast():
    grid, M, keep, dbeg, dcnt = _plan(1, 32, 8, 32768, 128, 8, "contiguous", True, -1, SKEW)
    slow = [x for x in range(8) if SKEW[x] < 0.99]
    fast = [x for x in range(8) if SKEW[x] > 1.01]
    assert all(keep[x] < M for x in slow) and all(dcnt[x] == 0 for x in slow)
    assert all(keep[x] == M for x in fast) and all(dcnt[x] > 0 for x in fast)
    assert keep[7] < keep[3] < keep[1] < M  # slower XCDs give more away
    assert dcnt[4] > dcnt[2]                # the fastest takes the most


def test_xcd_plan_keeps_uniform_items():
    # 16K tokens non-causal: every item is the same size, 8 per CU, so moving a
    # few items would only lengthen some CU's list; the split stays fixed
    grid, M, keep, dbeg, dcnt = _plan(1, 32, 32, 16384, 128, 8, "contiguous", False, -1, SKEW)
    assert keep == [M] * 8 and dcnt == [0] * 8 and grid == 8 * M


def test_xcd_plan_not_split():
    # fewer than 64 items per XCD, fp32 inputs (vector kernel), head dim 16
    assert _plan(1, 4, 2, 1024, 128, 4, "contiguous", True)[0] == 0
    assert _plan(1, 32, 8, 32768, 128, 8, "contiguous", True, dtype=torch.float32)[0] == 0
    assert _plan(1, 32, 8, 32768, 16, 8, "contiguous", True)[0] == 0


def test_xcd_plan_rejects_bad_arguments():
    with pytest.raises(ValueError, match="speeds"):
        _plan(1, 32, 8, 32768, 128, 8, "contiguous", True, -1, [1, 1, 1, 0, 1, 1, 1, 1])
    with pytest.raises(ValueError):
        _plan(1, 32, 8, 32768, 128, 7, "contiguous", True)          # S % N != 0
    with pytest.raises(ValueError):
        _plan(1, 32, 8, 32768, 128, 8, "contiguous", True, device=8)


def test_xcd_speeds_error_paths(lib):
    sp = (ctypes.c_float * 8)(*([1.0] * 8))
    n = ctypes.c_int(0)
    expect(lib.ra_xcd_speeds(sp, ctypes.byref(n), 3), capi.RA_ERR_ENUM, "set must be 0, 1 or 2")
    expect(lib.ra_xcd_speeds(sp, ctypes.byref(n), -1), capi.RA_ERR_ENUM, "set must be 0, 1 or 2")
    if torch.cuda.device_count() == 0:  # reading or setting the estimate needs a device
        expect(lib.ra_xcd_speeds(sp, ctypes.byref(n), 0), capi.RA_ERR_HIP, "no current HIP device")
