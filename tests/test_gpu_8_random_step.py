"""Seeded random sequences of ra_block_step calls against the fp64 oracle:
random key blocks (lengths 1 to 200, ragged), random global positions (any
order, repeats allowed, some queries seeing no key at all), causal or not,
every head dim, both dtypes and 1 to 8 query heads per key/value head.  The
state is folded block by block and finalized; the result must equal full
attention over the union of the blocks with the same positions."""

import zlib

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
from oracle import attention as O1
from gpu_helpers import check, log, rand

pytestmark = pytest.mark.gpu


def _draw_cases(n, seed=4049, budget=1.5e8):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = "bf16" if rng.random() < 0.7 else "fp32"
        D = int(rng.choice([8, 16, 32, 64, 128]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.choice([1, 2]))
        Sq = int(rng.integers(1, 400))
        nblk = int(rng.integers(1, 6))
        lens = tuple(int(x) for x in rng.integers(1, 201, size=nblk))
        causal = bool(rng.random() < 0.6)
        if B * Hkv * G * Sq * sum(lens) * D > budget:
            continue
        cases.append((dtype, B, Hkv * G, Hkv, D, Sq, lens, causal))
    return cases


CASES = _draw_cases(30)


@pytest.mark.parametrize(
    "case", CASES,
    ids=lambda c: "{}_B{}_H{}x{}_D{}_Sq{}_blocks{}_{}".format(
        c[0], c[1], c[2], c[3], c[4], c[5], "-".join(map(str, c[6])),
        "causal" if c[7] else "full"))
def test_random_steps(case):
    dtype_name, B, Hq, Hkv, D, Sq, lens, causal = case
    dtype = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    log(f"random steps {case}")
    seed = zlib.crc32(repr(case).encode()) % (2 ** 31)
    rng = np.random.default_rng(seed)
    Sk = sum(lens)
    q = rand((B, Hq, Sq, D), seed, dtype)
    k = rand((B, Hkv, Sk, D), seed + 1, dtype)
    v = rand((B, Hkv, Sk, D), seed + 2, dtype)
    # positions drawn from a range a little wider than the keys, with repeats;
    # the smallest query position lies below every key (that row sees nothing
    # under the causal mask)
    span = Sk + Sq
    kpos = rng.integers(0, span, size=Sk).astype(np.int32)
    qpos = rng.integers(0, span, size=Sq).astype(np.int32)
    qpos[int(rng.integers(0, Sq))] = -1
    mask = ra.RA_MASK_CAUSAL if causal else ra.RA_MASK_NONE
    st = ra.State(B, Hq, Sq, D)
    ra.ra_state_init(st)
    qd = q.cuda()
    qp = torch.from_numpy(qpos).cuda()
    a = 0
    for n in lens:
        kb = k[:, :, a:a + n].contiguous().cuda()
        vb = v[:, :, a:a + n].contiguous().cuda()
        kp = torch.from_numpy(kpos[a:a + n].copy()).cuda()
        ra.ra_block_step(qd, kb, vb, qp, kp, mask, st)
        a += n
    out = torch.empty((B, Hq, Sq, D), dtype=dtype, device="cuda")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    ra.ra_finalize(st, out, lse)
    torch.cuda.synchronize()
    ro, rl = O1.full_attention(q, k, v, q_pos=qpos, k_pos=kpos, causal=causal)
    check(out, lse, ro, rl, dtype, f"{case}")
