"""Vocab-parallel cross-entropy (ra_vocab_ce*, HIP) against the oracle's
three shard steps (oracle/vocab_ce.py).

Tolerances are derived from the fp32 arithmetic of the kernels (logits are
exact in fp32, so m and the target logit are exact):
  - each exponential is exp2(fma(z, log2 e, -m log2 e)); the rounded shift
    and the FMA put at most 2^-24 (2 |m| log2 e + |z - m| log2 e) on its
    exponent, the exp2 one more ulp;
  - a thread adds about V_loc / 256 terms in sequence, then 8 + log2(t)
    tree levels merge the partial sums;
so log Z, lse and the loss are off by at most 2^-24 (3 |m| + 64 + V_loc / 256
+ 16) plus half an ulp of the result; the tests allow twice that.  The
gradient adds one rounding of the output (bf16: half an ulp, 2^-9 relative).
"""

import math

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
from oracle import vocab_ce as O4
from gpu_helpers import log, to_np

pytestmark = pytest.mark.gpu


def make(N, V, dtype, seed, sigma=3.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    z = (torch.randn((N, V), generator=g) * sigma).to(dtype)
    tg = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    return z, tg


def set_targets(tg, V, t):
    """Targets on shard boundaries and outside the vocab in the first rows."""
    V_loc = V // t
    special = [0, V - 1, V_loc - 1, V_loc, -1, V, min(2 * V_loc, V - 1)]
    for i, x in enumerate(special[:len(tg)]):
        tg[i] = x
    return tg


def loss_tol(m, V_loc, value):
    m = np.abs(np.asarray(m, dtype=np.float64))
    ulp = np.spacing(np.abs(np.asarray(value, dtype=np.float32))).astype(np.float64)
    return 2.0 * (2.0 ** -24 * (3.0 * m + 64.0 + V_loc / 256.0 + 16.0) + 0.5 * ulp)


def check_rows(got, want, tol, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite rows differ"
    bad = err[fin] > np.broadcast_to(tol, want.shape)[fin]
    log(f"  {what}: max err {float(err[fin].max(initial=0)):.2e}, over bound {int(bad.sum())}")
    assert not bad.any(), f"{what}: max err {float(err[fin].max())}"


CASES = [
    # N, V, t, dtype
    (64, 4096, 8, torch.bfloat16),
    (33, 4096, 4, torch.float32),
    (40, 1000, 8, torch.bfloat16),   # V_loc = 125: shards off 16-byte boundaries
    (17, 999, 3, torch.float32),     # V_loc = 333
    (8, 50000, 1, torch.bfloat16),   # one shard
]


@pytest.mark.parametrize("N,V,t,dtype", CASES)
def test_vocab_ce_whole(N, V, t, dtype):
    log(f"vocab ce N={N} V={V} t={t} {dtype}")
    z, tg = make(N, V, dtype, 601 + V + t)
    tg = set_targets(tg, V, t)
    rl, rmean, rlse = O4.vocab_parallel(z, tg.numpy(), t)
    zg, tgg = z.cuda(), tg.cuda()
    loss = torch.empty(N, dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    ra.ra_vocab_ce(zg, tgg, t, loss, mean, lse)
    torch.cuda.synchronize()
    m = z.float().numpy().max(axis=1)
    check_rows(to_np(lse), rlse, loss_tol(m, V // t, rlse), "lse")
    check_rows(to_np(loss), rl, loss_tol(m, V // t, rl), "loss")
    tm = float(np.max(loss_tol(m, V // t, rl))) + 2.0 ** -24 * math.log2(N + 1) * abs(rmean) * 4
    em = abs(float(mean.item()) - rmean)
    log(f"  mean: err {em:.2e} (bound {tm:.2e})")
    assert em <= tm
    # deterministic: same bits on a second call
    loss2 = torch.empty_like(loss)
    mean2 = torch.empty_like(mean)
    ra.ra_vocab_ce(zg, tgg, t, loss2, mean2)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2) and torch.equal(mean, mean2)


@pytest.mark.parametrize("N,V,t,dtype", CASES[:4])
def test_vocab_ce_shards_then_combine(N, V, t, dtype):
    """ra_vocab_ce_shard on each column slice (row stride V), then
    ra_vocab_ce_combine, against the oracle's per-shard statistics."""
    log(f"vocab ce shards N={N} V={V} t={t} {dtype}")
    z, tg = make(N, V, dtype, 611 + V + t)
    tg = set_targets(tg, V, t)
    zg, tgg = z.cuda(), tg.cuda()
    V_loc = V // t
    m = torch.empty((t, N), dtype=torch.float32, device="cuda")
    s = torch.empty_like(m)
    p = torch.empty_like(m)
    for k in range(t):
        ra.ra_vocab_ce_shard(zg[:, k * V_loc:(k + 1) * V_loc], tgg, k * V_loc, m[k], s[k], p[k])
    torch.cuda.synchronize()
    for k in range(t):
        om, os_, op = O4.shard_stats(z[:, k * V_loc:(k + 1) * V_loc], tg.numpy(), k * V_loc)
        assert np.array_equal(to_np(m[k]), om), f"shard {k}: row max differs"
        assert np.array_equal(to_np(p[k]), op), f"shard {k}: target logit differs"
        rel = np.abs(to_np(s[k]) - os_) / os_
        bound = 2.0 * 2.0 ** -24 * (3.0 * np.abs(om) + 64.0 + V_loc / 256.0 + 16.0)
        assert np.all(rel <= bound), f"shard {k}: sum rel err {float(rel.max())}"
    loss = torch.empty(N, dtype=torch.float32, device="cuda")
    ra.ra_vocab_ce_combine(m, s, p, loss)
    torch.cuda.synchronize()
    rl, _, _ = O4.vocab_parallel(z, tg.numpy(), t)
    check_rows(to_np(loss), rl, loss_tol(z.float().numpy().max(axis=1), V_loc, rl), "combined loss")


@pytest.mark.parametrize("N,V,t,dtype", CASES[:4])
def test_vocab_ce_grad(N, V, t, dtype):
    """Gradient of the mean loss per shard against the oracle's
    softmax - onehot (scale 1/N)."""
    log(f"vocab ce grad N={N} V={V} t={t} {dtype}")
    z, tg = make(N, V, dtype, 621 + V + t)
    tg = set_targets(tg, V, t)
    zg, tgg = z.cuda(), tg.cuda()
    V_loc = V // t
    loss = torch.empty(N, dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    ra.ra_vocab_ce(zg, tgg, t, loss, mean, lse)
    grad = torch.empty_like(zg)
    for k in range(t):
        ra.ra_vocab_ce_grad(zg[:, k * V_loc:(k + 1) * V_loc], tgg, lse, k * V_loc, 1.0 / N,
                            grad[:, k * V_loc:(k + 1) * V_loc])
    torch.cuda.synchronize()
    ref = O4.ce_grad(z, tg.numpy(), 1.0 / N)
    got = to_np(grad)
    from scipy.special import softmax
    p = softmax(z.double().numpy(), axis=1) / N
    # lse error (loss_tol) moves every p by that much relative; bf16 rounds once
    lt = loss_tol(z.float().numpy().max(axis=1), V_loc, to_np(lse))[:, None]
    tol = 2.0 * p * lt + np.abs(ref) * (2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -22) + 1e-30
    bad = np.abs(got - ref) > tol
    log(f"  grad: max err {float(np.abs(got - ref).max()):.2e}, over bound {int(bad.sum())}")
    assert not bad.any()


def test_vocab_ce_full_size():
    """8192 rows x a 128,256-entry vocabulary (Llama-3's) in bf16 over 8
    shards: every row's loss against the oracle on 64 sampled rows, the
    mean against the fp64 mean of the GPU's own rows, and the gradient of
    the sampled rows."""
    N, V, t = 8192, 128256, 8
    log(f"vocab ce full size N={N} V={V} t={t}")
    g = torch.Generator(device="cuda")
    g.manual_seed(631)
    zg = (torch.randn((N, V), generator=g, device="cuda") * 3.0).to(torch.bfloat16)
    tgg = torch.randint(0, V, (N,), generator=g, device="cuda", dtype=torch.int64)
    loss = torch.empty(N, dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    ra.ra_vocab_ce(zg, tgg, t, loss, mean, lse)
    grad = torch.empty_like(zg)
    ra.ra_vocab_ce_grad(zg, tgg, lse, 0, 1.0 / N, grad)
    torch.cuda.synchronize()
    rows = np.random.default_rng(632).choice(N, 64, replace=False)
    zs = zg[rows].cpu()
    ts = tgg[rows].cpu().numpy()
    rl, _, _ = O4.vocab_parallel(zs, ts, t)
    check_rows(to_np(loss)[rows], rl, loss_tol(zs.float().numpy().max(axis=1), V // t, rl),
               "sampled loss")
    lg = to_np(loss)
    assert abs(float(mean.item()) - lg.mean()) <= 1e-6 * abs(lg.mean()) + 1e-6
    ref = O4.ce_grad(zs, ts, 1.0 / N)
    got = to_np(grad[rows])
    tol_p = 2.0 * (np.abs(ref) + 1.0 / N) * loss_tol(zs.float().numpy().max(axis=1), V, rl)[:, None]
    bad = np.abs(got - ref) > np.abs(ref) * 2.0 ** -8 + tol_p
    log(f"  sampled grad: over bound {int(bad.sum())}")
    assert not bad.any()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_vocab_ce_special_values(dtype):
    """Rows with -inf logits (a whole shard of them, or all but the target),
    a NaN logit and a +inf logit, against the oracle: an empty shard adds
    nothing, a NaN or +inf logit makes the row's loss NaN."""
    N, V, t = 6, 64, 4
    log(f"vocab ce special values {dtype}")
    z, tg = make(N, V, dtype, 641)
    z = z.float()
    tg[0] = 37
    z[0] = -float("inf")
    z[0, 37] = 1.5                  # only the target is finite: loss 0, lse 1.5
    z[1, 0:16] = -float("inf")      # shard 0 empty
    z[2, 55] = float("nan")         # NaN in shard 3
    z[3, 20] = float("inf")         # +inf in shard 1
    z = z.to(dtype)
    rl, _, rlse = O4.vocab_parallel(z, tg.numpy(), t)
    loss = torch.empty(N, dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    ra.ra_vocab_ce(z.cuda(), tg.cuda(), t, loss, mean, lse)
    torch.cuda.synchronize()
    gl, gs = to_np(loss), to_np(lse)
    assert np.array_equal(np.isnan(gl), np.isnan(rl)), (gl, rl)
    assert np.isnan(gl[2]) and np.isnan(gl[3])
    assert gl[0] == 0.0 and gs[0] == 1.5
    fin = np.isfinite(rl)
    m = np.nan_to_num(z.float().numpy(), nan=0.0, posinf=0.0, neginf=0.0).max(axis=1)
    check_rows(gl[fin], rl[fin], loss_tol(m[fin], V // t, rl[fin]), "finite rows")
    assert np.isnan(float(mean.item()))  # the mean of rows that include NaN
