"""ra_ring (the whole simulated ring, and one device's share) against the
fp64 oracle, element by element, at sizes the oracle finishes in seconds."""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
import workloads
from oracle import attention as O1
from oracle import layouts as OL
from gpu_helpers import check, gpu, log, rand, to_np, maxerr

pytestmark = pytest.mark.gpu

LAYOUTS = ["contiguous", "striped", "zigzag"]


def run_ring(q, k, v, N, layout, causal, device=-1):
    qd, kd, vd = gpu(q, k, v)
    out, lse = ra.ring_attention(qd, kd, vd, N, layout, causal, device)
    torch.cuda.synchronize()
    return out, lse


def test_tiny_case():
    """The pages' 4 devices x 3 tokens x d=8 case (fp32, non-causal)."""
    q, k, v = workloads.workload_inputs("tiny")
    out, lse = run_ring(q, k, v, 4, "contiguous", False)
    ro, rl = O1.full_attention(q, k, v)
    check(out, lse, ro, rl, torch.float32, "tiny N=4 blk=3 d=8")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout,N", [("contiguous", 4), ("striped", 4), ("zigzag", 2),
                                      ("zigzag", 3), ("contiguous", 1), ("striped", 12)])
def test_tiny_shapes_fp32(layout, N, causal):
    q, k, v = workloads.workload_inputs("tiny")
    out, lse = run_ring(q, k, v, N, layout, causal)
    ro, rl = O1.full_attention(q, k, v, causal=causal)
    check(out, lse, ro, rl, torch.float32, f"tiny {layout} N={N} causal={causal}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
def test_m23_fp32_tensors(layout, causal):
    """fp32 (2, 4, 96, 32) from torch.manual_seed(0), 8 devices (the first
    page's exactness demo), every layout."""
    torch.manual_seed(0)
    q, k, v = (torch.randn(2, 4, 96, 32) for _ in range(3))
    out, lse = run_ring(q, k, v, 8, layout, causal)
    ro, rl = O1.full_attention(q, k, v, causal=causal)
    check(out, lse, ro, rl, torch.float32, f"(2,4,96,32) {layout} causal={causal}")


@pytest.mark.parametrize("D", [8, 16, 32, 64, 128])
def test_fp32_head_dims(D):
    q = rand((1, 4, 80, D), 1, torch.float32)
    k = rand((1, 2, 80, D), 2, torch.float32)
    v = rand((1, 2, 80, D), 3, torch.float32)
    for layout in LAYOUTS:
        out, lse = run_ring(q, k, v, 4, layout, True)
        ro, rl = O1.full_attention(q, k, v, causal=True)
        check(out, lse, ro, rl, torch.float32, f"fp32 D={D} {layout}")


# bf16: matrix-core kernel for D in {32, 64, 128}, vector kernel for 8, 16.
BF16_CASES = [
    # (B, Hq, Hkv, S, N, D)
    (1, 4, 2, 1024, 4, 128),   # one 256-row query tile and four 64-key tiles per block
    (1, 4, 1, 600, 3, 128),    # ragged: blocks of 200 (not a multiple of 64)
    (2, 2, 2, 512, 8, 64),     # batch 2, MHA, blocks of 64
    (1, 8, 2, 384, 2, 32),     # D = 32
    (1, 2, 1, 136, 4, 16),     # vector kernel (bf16, D = 16), ragged blocks of 34
    (1, 2, 2, 96, 3, 8),       # vector kernel (bf16, D = 8)
    (1, 4, 4, 4096, 8, 128),   # blocks of 512, many tiles
    (1, 4, 2, 1200, 4, 128),   # blocks of 300: 256-row query tiles with a ragged second tile
    (1, 2, 1, 1020, 4, 128),   # blocks of 255: the largest block on 128-row query tiles
    (2, 8, 1, 2048, 4, 128),   # batch 2, 8 query heads per key/value head, blocks of 512
]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "B{}_H{}x{}_S{}_N{}_D{}".format(*c))
def test_bf16_ring(case, causal, layout):
    B, Hq, Hkv, S, N, D = case
    if layout == "zigzag" and S % (2 * N):
        pytest.skip("zigzag needs S % 2N == 0")
    log(f"bf16 ring {case} causal={causal} {layout}")
    seed = sum(case) + 7 * causal
    q = rand((B, Hq, S, D), seed, torch.bfloat16)
    k = rand((B, Hkv, S, D), seed + 1, torch.bfloat16)
    v = rand((B, Hkv, S, D), seed + 2, torch.bfloat16)
    out, lse = run_ring(q, k, v, N, layout, causal)
    ro, rl = O1.full_attention(q, k, v, causal=causal)
    check(out, lse, ro, rl, torch.bfloat16, f"{case} {layout} causal={causal}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_device_share(layout, dtype):
    """device = p: p's query block in local order against all K/V blocks in
    device order (the one-GPU share of a real ring)."""
    B, Hq, Hkv, S, N, D = 1, 4, 2, 2048, 8, 128
    q = rand((B, Hq, S, D), 11, dtype)
    k = rand((B, Hkv, S, D), 12, dtype)
    v = rand((B, Hkv, S, D), 13, dtype)
    ro, rl = O1.full_attention(q, k, v, causal=True)
    kd = torch.from_numpy(OL.to_device_order(k.float().numpy(), N, layout, axis=2)).to(dtype)
    vd = torch.from_numpy(OL.to_device_order(v.float().numpy(), N, layout, axis=2)).to(dtype)
    for p in (0, 3, N - 1):
        pos = OL.device_positions(S, N, layout, p)
        qp = q[:, :, pos].contiguous()
        out, lse = run_ring(qp, kd, vd, N, layout, True, device=p)
        check(out, lse, ro[:, :, pos], rl[:, :, pos], dtype, f"share p={p} {layout} {dtype}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_constant_scores(dtype):
    """Q = 0: every row is the mean of its visible values and lse = ln #visible."""
    B, Hq, Hkv, S, N, D = 1, 2, 1, 512, 4, 128
    q = torch.zeros((B, Hq, S, D), dtype=dtype)
    k = rand((B, Hkv, S, D), 21, dtype)
    v = rand((B, Hkv, S, D), 22, dtype)
    vv = v[0, 0].double().numpy()
    mean = np.cumsum(vv, axis=0) / np.arange(1, S + 1)[:, None]
    for layout in LAYOUTS:
        out, lse = run_ring(q, k, v, N, layout, True)
        ro = np.broadcast_to(mean, (B, Hq, S, D))
        rl = np.broadcast_to(np.log(np.arange(1, S + 1)), (B, Hq, S))
        check(out, lse, ro, rl, dtype, f"Q=0 {layout}")


def test_single_visible_key():
    """Causal row at global position 0 sees only key 0: out = v_0, lse = s_00."""
    B, Hq, Hkv, S, N, D = 1, 2, 2, 256, 4, 128
    q = rand((B, Hq, S, D), 31, torch.bfloat16)
    k = rand((B, Hkv, S, D), 32, torch.bfloat16)
    v = rand((B, Hkv, S, D), 33, torch.bfloat16)
    for layout in LAYOUTS:
        out, lse = run_ring(q, k, v, N, layout, True)
        for h in range(Hq):
            s00 = float(q[0, h, 0].double() @ k[0, h, 0].double()) / np.sqrt(D)
            assert maxerr(to_np(out[0, h, 0]), v[0, h, 0].double().numpy()) <= 2e-2 / 8
            assert abs(float(lse[0, h, 0]) - s00) <= 1e-5


def test_layout_invariance_gpu():
    """Striped / zigzag causal output equals contiguous causal output (GPU vs GPU)."""
    B, Hq, Hkv, S, N, D = 1, 4, 2, 2048, 8, 128
    q = rand((B, Hq, S, D), 41, torch.bfloat16)
    k = rand((B, Hkv, S, D), 42, torch.bfloat16)
    v = rand((B, Hkv, S, D), 43, torch.bfloat16)
    base = run_ring(q, k, v, N, "contiguous", True)
    for layout in ("striped", "zigzag"):
        o, l_ = run_ring(q, k, v, N, layout, True)
        eo = maxerr(to_np(o), to_np(base[0]))
        el = maxerr(to_np(l_), to_np(base[1]))
        log(f"  {layout} vs contiguous: out {eo:.2e} lse {el:.2e}")
        assert eo <= 2e-2 and el <= 1e-3


def test_deterministic():
    B, Hq, Hkv, S, N, D = 1, 4, 2, 1024, 4, 128
    q = rand((B, Hq, S, D), 51, torch.bfloat16)
    k = rand((B, Hkv, S, D), 52, torch.bfloat16)
    v = rand((B, Hkv, S, D), 53, torch.bfloat16)
    a = run_ring(q, k, v, N, "zigzag", True)
    b = run_ring(q, k, v, N, "zigzag", True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
def test_score_jumps(layout, causal):
    """Keys in every third 64-key tile are scaled by 30, so a row's scores
    jump by far more than 2^64 in base-2 units between tiles in every ring
    order: the kernels must rescale the running state mid-stream (and never
    let an exponential overflow).  The peaked rows make each output close to
    a single value row, so V is drawn with standard deviation 1/4: bf16
    rounding of an output near 4 alone costs up to 0.016 of the absolute
    tolerance, while a wrong rescale shows up at the size of V itself."""
    B, Hq, Hkv, S, N, D = 1, 4, 2, 1536, 4, 128
    q = rand((B, Hq, S, D), 61, torch.float32)
    k = rand((B, Hkv, S, D), 62, torch.float32)
    v = rand((B, Hkv, S, D), 63, torch.float32) * 0.25
    f = np.where((np.arange(S) // 64) % 3 == 2, 30.0, 1.0)
    k = k * torch.from_numpy(f).float()[None, None, :, None]
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    out, lse = run_ring(q, k, v, N, layout, causal)
    ro, rl = O1.full_attention(q, k, v, causal=causal)
    assert float(np.max(rl)) > 40.0  # some rows meet scores far above their earlier tiles
    check(out, lse, ro, rl, torch.bfloat16, f"score jumps {layout} causal={causal}")


def step_api_ring(q, k, v, N, layout):
    """The same causal ring through ra_block_step (one call per block, ring
    order, explicit positions) and ra_finalize; natural order in and out."""
    B, Hq, S, D = q.shape
    blk = S // N
    qd, kd, vd = gpu(q, k, v)
    out = torch.empty_like(qd)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    for p in range(N):
        qpos = OL.device_positions(S, N, layout, p)
        qi = qd[:, :, qpos].contiguous()
        st = ra.State(B, Hq, blk, D)
        ra.ra_state_init(st)
        qp = torch.from_numpy(qpos.astype(np.int32)).cuda()
        for s in range(N):
            j = (p - s) % N
            kpos = OL.device_positions(S, N, layout, j)
            kp = torch.from_numpy(kpos.astype(np.int32)).cuda()
            ra.ra_block_step(qi, kd[:, :, kpos].contiguous(), vd[:, :, kpos].contiguous(), qp,
                             kp, ra.RA_MASK_CAUSAL, st)
        o = torch.empty_like(qi)
        l_ = torch.empty((B, Hq, blk), dtype=torch.float32, device="cuda")
        ra.ra_finalize(st, o, l_)
        out[:, :, qpos] = o
        lse[:, :, qpos] = l_
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 64)])
def test_very_negative_scores(layout, dtype, D):
    """Every score far below the exponential's range against a zero reference.

    Part 1: q = -c * 1, k = 1 gives the constant score s = -c sqrt(D) ~ -120
    (natural log), so exp(s) underflows in fp32 for every pair; the result is
    still exact: out = mean of the visible value rows, lse = s + ln(#visible).
    Part 2: random rows with q_0 = -c' k_0, so the first causal row's only
    visible score is ~ -110.  The whole ring (which starts without a reference)
    must agree with the oracle and with the step API (which takes row maxima)."""
    B, Hq, Hkv, S, N = 1, 4, 2, 1024, 4
    c = 10.625 if D == 128 else 13.25  # exact in bf16; s = -c * sqrt(D): -120.2, -106
    q = torch.full((B, Hq, S, D), -c, dtype=torch.float32)
    k = torch.ones((B, Hkv, S, D), dtype=torch.float32)
    v = rand((B, Hkv, S, D), 71, torch.float32)
    q, k, v = (t.to(dtype) for t in (q, k, v))
    out, lse = run_ring(q, k, v, N, layout, True)
    ro, rl = O1.full_attention(q, k, v, causal=True)
    s = -c * np.sqrt(D)
    assert s < -100
    n = np.arange(1, S + 1)
    assert np.allclose(rl[0, 0], s + np.log(n), atol=1e-9)  # the closed form, in the oracle too
    check(out, lse, ro, rl, dtype, f"constant score {s:.1f} {layout} D={D}")
    so, sl = step_api_ring(q, k, v, N, layout)
    check(so, sl, ro, rl, dtype, f"constant score {s:.1f}, step API, {layout} D={D}")

    q = rand((B, Hq, S, D), 72, torch.float32)
    k = rand((B, Hkv, S, D), 73, torch.float32)
    G = Hq // Hkv
    k = k.to(dtype).float()
    for h in range(Hq):
        k0 = k[0, h // G, 0]
        q[0, h, 0] = -(110.0 * np.sqrt(D) / float((k0 * k0).sum())) * k0
    q, k = q.to(dtype), k.to(dtype)
    out, lse = run_ring(q, k, v, N, layout, True)
    ro, rl = O1.full_attention(q, k, v, causal=True)
    assert float(rl[0, :, 0].max()) < -105
    check(out, lse, ro, rl, dtype, f"single key at ~-110 {layout} D={D}")
    so, sl = step_api_ring(q, k, v, N, layout)
    check(so, sl, ro, rl, dtype, f"single key at ~-110, step API, {layout} D={D}")
    eo = maxerr(to_np(out), to_np(so))
    log(f"  whole ring vs step API: out {eo:.2e}")
