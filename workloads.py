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
Every bf16 tensor is drawn as torch.randn in float32 from a CPU
torch.Generator seeded with the workload's seed (Q, then K, then V), then
rounded to bf16 (round-to-nearest-even).  Large tensors are drawn in chunks
of CHUNK_ROWS rows along the flattened [rows, D] view, in order, from the same
generator, so the draw is deterministic for a given seed and shape.
"""

import numpy as np
import torch

CHUNK_ROWS = 1 << 16

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


def randn(shape, gen, dtype=torch.bfloat16):
    """N(0,1) draw in float32 from `gen`, chunked by rows, rounded to `dtype`."""
    shape = tuple(int(s) for s in shape)
    D = shape[-1]
    rows = int(np.prod(shape[:-1]))
    out = torch.empty((rows, D), dtype=dtype)
    for r0 in range(0, rows, CHUNK_ROWS):
        r1 = min(rows, r0 + CHUNK_ROWS)
        out[r0:r1] = torch.randn((r1 - r0, D), generator=gen, dtype=torch.float32).to(dtype)
    return out.view(shape)


def qkv(B, Hq, Hkv, Sq, Sk, D, seed, dtype=torch.bfloat16):
    """Q [B,Hq,Sq,D], K, V [B,Hkv,Sk,D] on the CPU, drawn in that order."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    q = randn((B, Hq, Sq, D), gen, dtype)
    k = randn((B, Hkv, Sk, D), gen, dtype)
    v = randn((B, Hkv, Sk, D), gen, dtype)
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


def sample_rows(Hq, Sq, n_rows, seed, must_include=()):
    """Seeded (h, i) row sample: n_rows // Hq rows per head plus `must_include`.

    must_include: sequence indices every head includes (chunk first/last rows).
    Returns a sorted list of (h, i).
    """
    rng = np.random.default_rng(seed)
    per_head = max(1, n_rows // Hq)
    rows = []
    for h in range(Hq):
        fixed = sorted(set(int(i) for i in must_include))
        rest = per_head - len(fixed)
        pool = np.setdiff1d(np.arange(Sq), np.array(fixed, dtype=np.int64))
        pick = rng.choice(pool, size=max(0, rest), replace=False) if rest > 0 else []
        for i in sorted(fixed + [int(x) for x in pick])[:per_head]:
            rows.append((h, i))
    return rows
