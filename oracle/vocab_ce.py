"""O4: vocab-parallel cross-entropy, the second workload of the max-then-sum
softmax.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Definition ([DT2] "Vocab-parallel cross-entropy"): for logits z of shape
[N, V] and global target ids t (one per row), the loss of row r is
    loss_r = logsumexp(z_r) - z_r[t_r]
and the reported loss is the mean over rows.  The page computes it with the
vocab split into `t` contiguous shards of V_loc = V / t columns (rank k owns
columns [k V_loc, (k+1) V_loc)), in three steps:
    1. m   = max over shards of the shard's row max          (all-reduce MAX)
    2. Z   = sum over shards of sum_j exp(z_kj - m)           (all-reduce SUM)
    3. z_t = sum over shards of the shard's target logit, where a shard that
             does not own t_r contributes 0                   (all-reduce SUM)
    loss = log Z + m - z_t.
Its gradient with respect to the logits of the mean loss is
    (softmax(z_r) - onehot(t_r)) / N,
already split along the vocab like the logits.

Readings taken (the page is silent on them):
  - A target outside [0, V) is owned by no shard: its z_t is 0, as the
    page's mask makes it, so loss_r = logsumexp(z_r).
  - Logits are upcast exactly to fp64 (bf16 and fp32 both are exact in fp64).

Functions:
  cross_entropy_rows(z, target)   plain definition, per row (scipy's
                                  logsumexp of the row minus the target logit)
  vocab_parallel(z, target, t)    the page's three steps over t shards,
                                  per-row loss, the mean, and m + log Z
  shard_stats(z_shard, target, start)
                                  one shard's (row max, sum of exp(z - that
                                  max), owned target logit)
  ce_grad(z, target, scale)       scale * (softmax(z) - onehot(target))
"""

import numpy as np

from .attention import _as_f64


def _targets(target):
    return np.asarray(target, dtype=np.int64).reshape(-1)


def cross_entropy_rows(z, target):
    """loss_r = logsumexp(z_r) - z_r[target_r] (target_r outside [0, V): 0)."""
    from scipy.special import logsumexp

    z = _as_f64(z)
    t = _targets(target)
    V = z.shape[1]
    own = (t >= 0) & (t < V)
    zt = np.where(own, z[np.arange(len(t)), np.clip(t, 0, V - 1)], 0.0)
    return logsumexp(z, axis=1) - zt


def shard_stats(z_shard, target, start):
    """One shard's row max, sum of exp(z - row max) and owned target logit."""
    z = _as_f64(z_shard)
    t = _targets(target)
    V_loc = z.shape[1]
    m = z.max(axis=1)
    s = np.exp(z - m[:, None]).sum(axis=1)
    own = (t >= start) & (t < start + V_loc)
    pred = np.where(own, z[np.arange(len(t)), np.clip(t - start, 0, V_loc - 1)], 0.0)
    return m, s, pred


def vocab_parallel(z, target, t):
    """The page's three steps over t contiguous vocab shards.

    Returns (loss per row, mean loss, lse = m + log Z per row)."""
    z = _as_f64(z)
    tg = _targets(target)
    N, V = z.shape
    assert V % t == 0, "the page splits the vocab evenly (V_loc = V / t)"
    V_loc = V // t
    shards = [z[:, k * V_loc:(k + 1) * V_loc] for k in range(t)]
    # 1) global row max (all-reduce MAX over the shards' row maxima)
    m = np.max(np.stack([sh.max(axis=1) for sh in shards]), axis=0)
    # 2) global normaliser (all-reduce SUM of each shard's exp-sum against m)
    Z = np.sum(np.stack([np.exp(sh - m[:, None]).sum(axis=1) for sh in shards]), axis=0)
    # 3) the target logit: only the owning shard contributes
    preds = []
    for k, sh in enumerate(shards):
        start = k * V_loc
        own = (tg >= start) & (tg < start + V_loc)
        local = np.clip(tg - start, 0, V_loc - 1)
        preds.append(np.where(own, sh[np.arange(N), local], 0.0))
    pred = np.sum(np.stack(preds), axis=0)
    loss = np.log(Z) + m - pred
    return loss, float(loss.mean()), m + np.log(Z)


def ce_grad(z, target, scale):
    """scale * (softmax(z) - onehot(target)); a target outside [0, V) has no
    one-hot entry."""
    z = _as_f64(z)
    tg = _targets(target)
    N, V = z.shape
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    g = e / e.sum(axis=1, keepdims=True)
    own = (tg >= 0) & (tg < V)
    g[np.arange(N)[own], tg[own]] -= 1.0
    return g * scale
