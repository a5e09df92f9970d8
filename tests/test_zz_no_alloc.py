"""ra_vocab_ce_static (no workspace, the library's static per-GPU scratch)
against ra_vocab_ce (caller's workspace) through the C ABI: identical loss,
lse and mean on two calls in a row, the second with fewer rows and shards, so
the scratch still holds the first call's larger contents."""

import pytest
import torch

import blockwise_online_softmax_amd as ra
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _inputs(N, V, seed, dtype):
    g = torch.Generator(device="cpu").manual_seed(seed)
    z = (torch.randn((N, V), generator=g) * 3.0).to(dtype).cuda()
    tg = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    tg[::7] = V + 5  # targets outside the vocab: owned by no shard
    return z, tg.cuda()


def _run(fn, z, tg, t, **kw):
    N = z.shape[0]
    loss = torch.full((N,), float("nan"), device="cuda")
    lse = torch.full((N,), float("nan"), device="cuda")
    mean = torch.full((1,), float("nan"), device="cuda")
    fn(z, tg, t, loss, mean, lse, **kw)
    torch.cuda.synchronize()
    return loss, lse, mean


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_static_scratch_matches_workspace(dtype):
    for call, (N, V, t) in enumerate(((8192, 32768, 8), (1000, 6000, 3))):
        log(f"vocab CE static scratch, call {call}: N={N} V={V} t={t} {dtype}")
        z, tg = _inputs(N, V, 40 + call, dtype)
        a = _run(ra.ra_vocab_ce, z, tg, t)
        b = _run(ra.ra_vocab_ce_static, z, tg, t)
        for x, y, name in zip(a, b, ("loss", "lse", "mean")):
            assert torch.isfinite(x).all(), name
            assert torch.equal(x, y), (name, float((x - y).abs().max()))
        log(f"  identical: loss, lse, mean ({float(a[2]):.6f})")
