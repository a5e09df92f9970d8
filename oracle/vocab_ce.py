"""O4: vocab-parallel cross-entropy, the second workload of the max-then-sum
softmax.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Definition ([DT2] "Vocab-parallel cross-entropy"): for logits z of shape
[N, V] and global target ids t (one per row), the loss of row r is
    loss_r = logsumexp(z_r) - z_r[t_r]
and the reported loss is the mean over rows.  The page computes it with the
vocab split into `t` contiguous shards of V_loc = V / t columns (rank k owns
columns [k V_loc, (k+1) V_loc)): the global row max, the sum of the shards'
exponentials against it, and the target logit (contributed by the shard that
owns it, 0 elsewhere), each reduced across ranks; the loss is log Z + max -
target logit.  Here the shards' (max, sum) pairs are merged in the log domain
instead, which gives the same log Z.
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
  vocab_parallel(z, target, t)    over t shards: per-shard statistics merged
                                  by log-sum-exp; per-row loss, the mean, log Z
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
    """One shard's row max, sum of exp(z - row max) and owned target logit.
    A row whose logits are all -inf has max -inf and sum 0 (a +inf or NaN
    logit leaves the sum NaN)."""
    z = _as_f64(z_shard)
    t = _targets(target)
    V_loc = z.shape[1]
    m = z.max(axis=1)
    s = np.exp(z - np.where(m == -np.inf, 0.0, m)[:, None]).sum(axis=1)
    own = (t >= start) & (t < start + V_loc)
    pred = np.where(own, z[np.arange(len(t)), np.clip(t - start, 0, V_loc - 1)], 0.0)
    return m, s, pred


def vocab_parallel(z, target, t):
    """The loss over t contiguous vocab shards, from per-shard statistics.

    Each shard is reduced on its own (shard_stats).  Its log-normaliser,
    log sum_j exp(z_j) over its columns, is m_k + log s_k; the log-normaliser
    of a union of shards is the log-sum-exp of theirs (an associative merge,
    so the order of the shards does not matter), and the target logit is the
    sum of the owned ones (at most one shard owns a target).
    Returns (loss per row, mean loss, lse = log Z per row)."""
    z = _as_f64(z)
    tg = _targets(target)
    N, V = z.shape
    assert V % t == 0, "the page splits the vocab evenly (V_loc = V / t)"
    V_loc = V // t
    stats = [shard_stats(z[:, k * V_loc:(k + 1) * V_loc], tg, k * V_loc) for k in range(t)]
    with np.errstate(divide="ignore"):  # log 0 = -inf for a shard of -inf logits
        log_z = [m + np.log(s) for m, s, _ in stats]
    lse = log_z[0]
    for lz in log_z[1:]:
        lse = np.logaddexp(lse, lz)
    pred = np.sum(np.stack([p for _, _, p in stats]), axis=0)
    loss = lse - pred
    return loss, float(loss.mean()), lse


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
