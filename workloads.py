"""Seeded synthetic inputs for the ring-attention workloads.

This module holds no attention arithmetic: it only fixes shapes and draws
random tensors, so that the oracle and the HIP path see identical inputs.

Workloads (sizes from the pages' cases and a Llama-3-8B attention layer:
32 query heads, 8 key/value heads, head dim 128):
  tiny      4 devices x 3 tokens, head dim 8, 1 head, fp32, non-causal.  Drawn
            exactly as the numpy simulation on the page "Explain ring
            attention..." (section "The ring") draws it:
            numpy default_rng(1), then Q, K, V = rng.normal(size=(12, 8)).
  mha16k    non-causal, 8 blocks of 2048 (S = 16384), 32/32 heads, D 128, bf16.
  gqa32k    causal contiguous, 8 blocks of 4096 (S = 32768), 32/8 heads, bf16.
  gqa64k    causal, S = 65536, N = 8, 32/8 heads, bf16; run under contiguous,
            striped and zigzag layouts on the same tensors.
  share1m   one device's zigzag share of S = 1,048,576 over N = 8: 131072
            queries (device 0) against all 8 K/V blocks in device order,
            causal, 32/8 heads, bf16.
Every bf16 tensor of the large workloads is drawn as N(0,1) float32 with
numpy and rounded to bf16 (round-to-nearest-even): tensor t (0 = Q, 1 = K,
2 = V) of a workload with seed s uses numpy.random.SeedSequence([s, t]); its
flattened elements are cut into chunks of CHUNK elements, chunk c is filled
by Generator(PCG64(child c of that sequence)).standard_normal(float32).  The
draw is deterministic for any number of worker threads.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

CHUNK = 1 << 22
THREADS = min(16, os.cpu_count() or 1)

WORKLOADS = {
    "tiny": dict(B=1, Hq=1, Hkv=1, S=12, N=4, D=8, dtype="f32", causal=False,
                 layouts=("contiguous",), seed=1),
    "mha16k": dict(B=1, Hq=32, Hkv=32, S=16384, N=8, D=128, dtype="bf16",
                   causal=False, layouts=("contiguous",), seed=2),
    "gqa32k": dict(B=1, Hq=32, Hkv=8, S=32768, N=8, D=128, dtype="bf16",
                   causal=True, layouts=("contiguous",), seed=3),
    "gqa64k": dict(B=1, Hq=32, Hkv=8, S=65536, N=8, D=128, dtype="bf16",
                   causal=True, layouts=("contiguous", "striped", "zigzag"), seed=4),
    "share1m": dict(B=1, Hq=32, Hkv=8, S=1048576, N=8, D=128, dtype="bf16",
                    causal=True, layouts=("zigzag",), seed=5, device=0),
}


def tiny_inputs():
    """The page's tiny case: float64 arrays Q, K, V of shape (12, 8)."""
    rng = np.random.default_rng(1)
    N, blk, d = 4, 3, 8
    Q, K, V = (rng.normal(size=(N * blk, d)) for _ in range(3))
    return Q, K, V


def randn(shape, seed, index, dtype=torch.bfloat16):
    """N(0,1) tensor of `shape`: float32 chunks from spawned PCG64 streams, rounded to dtype."""
    shape = tuple(int(x) for x in shape)
    n = int(np.prod(shape))
    nchunks = (n + CHUNK - 1) // CHUNK
    kids = np.random.SeedSequence([int(seed), int(index)]).spawn(nchunks)
    out = torch.empty(n, dtype=dtype)

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        x = np.random.Generator(np.random.PCG64(kids[c])).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi].copy_(torch.from_numpy(x))

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(fill, range(nchunks)))
    return out.view(shape)


def qkv(B, Hq, Hkv, Sq, Sk, D, seed, dtype=torch.bfloat16):
    """Q [B,Hq,Sq,D], K, V [B,Hkv,Sk,D] on the CPU (tensor indices 0, 1, 2)."""
    q = randn((B, Hq, Sq, D), seed, 0, dtype)
    k = randn((B, Hkv, Sk, D), seed, 1, dtype)
    v = randn((B, Hkv, Sk, D), seed, 2, dtype)
    return q, k, v


def workload_inputs(name):
    """CPU tensors for a named workload.

    Returns (q, k, v).  For 'share1m' q is the device-0 query share
    [1, 32, 131072, 128] in that device's local order and k, v are the full
    [1, 8, 1048576, 128] sequences in device order.
    """
    w = WORKLOADS[name]
    if name == "tiny":
        Q, K, V = tiny_inputs()
        f = lambda a: torch.from_numpy(a.astype(np.float32)).view(1, 1, 12, 8)
        return f(Q), f(K), f(V)
    Sq = w["S"] // w["N"] if name == "share1m" else w["S"]
    return qkv(w["B"], w["Hq"], w["Hkv"], Sq, w["S"], w["D"], w["seed"])


def sample_rows(Hq, Sq, per_head, seed, strata=None, include_ends=False):
    """Seeded sample of (h, i) query rows: `per_head` rows for every head.

    strata: index ranges (lo, hi) that share a head's rows equally (default
    the whole range); include_ends makes every stratum contribute its first
    and last index.  Returns a list of (h, i) sorted by head, then index.
    """
    rng = np.random.default_rng(seed)
    strata = strata or [(0, Sq)]
    share = max(1, per_head // len(strata))
    rows = []
    for h in range(Hq):
        picks = set()
        for lo, hi in strata:
            fixed = {lo, hi - 1} if include_ends else set()
            pool = np.setdiff1d(np.arange(lo, hi), np.array(sorted(fixed), dtype=np.int64))
            extra = rng.choice(pool, size=max(0, share - len(fixed)), replace=False)
            picks |= fixed | set(int(x) for x in extra)
        rows += [(h, i) for i in sorted(picks)]
    return rows
