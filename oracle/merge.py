"""O3: merge of two partial results over disjoint key sets.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[M23] "The Math: One Block at a Time" notes that the fold does not depend on
the order in which blocks arrive.  A running state (m, l, o) built from one
key set therefore folds into another exactly like one more block: the second
state's max plays the part of the block max, its denominator and output the
part of the block's sums.  With m = max(m_a, m_b):
    l = l_a exp(m_a - m) + l_b exp(m_b - m)
    o = o_a exp(m_a - m) + o_b exp(m_b - m)
Reading taken: a side with m = -inf (it saw no key) contributes nothing, and
a row empty on both sides stays empty (m = -inf, l = 0, o = 0), as in the
guarded fold of ring.py.

For finalized results (out, lse) the same step is the log-sum-exp merge that
[DT2] "Vocab-parallel cross-entropy" runs across vocab shards: take the
global max m of the shards, sum the shards' normalisers Z rescaled to it, and
logsumexp = m + log Z.  Here the shard normalisers are exp(lse_a - m) and
exp(lse_b - m), and each side's output is weighted by its share of Z:
    lse = m + log(exp(lse_a - m) + exp(lse_b - m))
    out = out_a exp(lse_a - lse) + out_b exp(lse_b - lse)
A row with lse = -inf on both sides gets out = 0, lse = -inf.
"""

import numpy as np

from .attention import _as_f64


def _side_weight(x, ref):
    """exp(x - ref) with 0 where x is -inf (also where ref is -inf)."""
    finite = np.isfinite(x)
    return np.where(finite, np.exp(np.where(finite, x, 0.0) - np.where(finite, ref, 0.0)), 0.0)


def merge_states(a, b):
    """Merge running states a = (m, l, o) and b over disjoint key sets."""
    ma, la, oa = (_as_f64(t) for t in a)
    mb, lb, ob = (_as_f64(t) for t in b)
    m = np.maximum(ma, mb)
    wa = _side_weight(ma, m)
    wb = _side_weight(mb, m)
    l = la * wa + lb * wb
    o = oa * wa[..., None] + ob * wb[..., None]
    return (m, l, o)


def merge_outputs(out_a, lse_a, out_b, lse_b):
    """Merge finalized (out, lse) pairs over disjoint key sets."""
    out_a, lse_a, out_b, lse_b = (_as_f64(t) for t in (out_a, lse_a, out_b, lse_b))
    m = np.maximum(lse_a, lse_b)
    z = _side_weight(lse_a, m) + _side_weight(lse_b, m)
    seen = z > 0
    lse = np.where(seen, m + np.log(np.where(seen, z, 1.0)), -np.inf)
    ref = np.where(seen, lse, 0.0)
    wa = np.where(seen, _side_weight(lse_a, ref), 0.0)
    wb = np.where(seen, _side_weight(lse_b, ref), 0.0)
    out = out_a * wa[..., None] + out_b * wb[..., None]
    return out, lse
