"""Seeded random shapes for ra_ring against the fp64 oracle: batch, heads and
grouping, head dim, ring size, block length (ragged and tiny included),
layout, causal or not, dtype, the whole ring and one device's share.  The
configurations are drawn once from a fixed seed, so every run checks the same
cases; each is small enough for the oracle to finish in well under a second."""

import zlib

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
from oracle import attention as O1
from oracle import layouts as OL
from gpu_helpers import check, gpu, log, rand

pytestmark = pytest.mark.gpu


def _draw_cases(n, seed=2026, budget=3.0e8):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = "bf16" if rng.random() < 0.7 else "fp32"
        D = int(rng.choice([8, 16, 32, 64, 128]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.choice([1, 2]))
        N = int(rng.integers(1, 9))
        layout = str(rng.choice(["contiguous", "striped", "zigzag"]))
        blk = int(rng.integers(1, 321))
        if layout == "zigzag" and blk % 2:
            blk += 1
        S = N * blk
        causal = bool(rng.random() < 0.6)
        # oracle work ~ B * Hq * S^2 * D
        if B * Hkv * G * S * S * D > budget:
            continue
        device = int(rng.integers(0, N))
        cases.append((dtype, B, Hkv * G, Hkv, S, N, D, layout, causal, device))
    return cases


CASES = _draw_cases(40)


@pytest.mark.parametrize(
    "case", CASES,
    ids=lambda c: "{}_B{}_H{}x{}_S{}_N{}_D{}_{}_{}_p{}".format(
        c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], "causal" if c[8] else "full", c[9]))
def test_random_ring(case):
    dtype_name, B, Hq, Hkv, S, N, D, layout, causal, p = case
    dtype = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    log(f"random ring {case}")
    seed = zlib.crc32(repr(case).encode()) % (2 ** 31)
    q = rand((B, Hq, S, D), seed, dtype)
    k = rand((B, Hkv, S, D), seed + 1, dtype)
    v = rand((B, Hkv, S, D), seed + 2, dtype)
    ro, rl = O1.full_attention(q, k, v, causal=causal)
    # the whole ring, natural order in and out
    qd, kd, vd = gpu(q, k, v)
    out, lse = ra.ring_attention(qd, kd, vd, N, layout, causal, -1)
    torch.cuda.synchronize()
    check(out, lse, ro, rl, dtype, f"{case} whole ring")
    # device p's share: its query block in local order, K/V in device order
    pos = OL.device_positions(S, N, layout, p)
    kdev = torch.from_numpy(OL.to_device_order(k.float().numpy(), N, layout, axis=2)).to(dtype)
    vdev = torch.from_numpy(OL.to_device_order(v.float().numpy(), N, layout, axis=2)).to(dtype)
    qp, kp, vp = gpu(q[:, :, pos].contiguous(), kdev, vdev)
    out_p, lse_p = ra.ring_attention(qp, kp, vp, N, layout, causal, p)
    torch.cuda.synchronize()
    check(out_p, lse_p, ro[:, :, pos], rl[:, :, pos], dtype, f"{case} share p={p}")
