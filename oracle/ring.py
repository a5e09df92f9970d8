"""O2: the blockwise online-softmax recurrence, run as a simulated ring.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Recurrence: [M23] "The Math: One Block at a Time".  Each query row keeps a
running max m, a running denominator l and an unnormalised output o.  When a
key/value block with scores s_ij = q_i . k_j / sqrt(d) arrives, the new
running max is the larger of m and the block's largest score; what is already
summed is rescaled by exp(m_old - m_new); the block adds exp(s_ij - m_new) to l
and exp(s_ij - m_new) v_j to o.  At the end out = o / l.  [RAQA] "The ring" runs the same loop in numpy
with m = -inf, l = 0, o = 0 as the start; [DT2] "Ring Attention" starts m at
-1e30 instead.  Reading taken: start at -inf and guard the case where no key
has been visible yet (m_new = -inf): then c = 1 and the block adds nothing,
which is what -1e30 gives for every row that sees at least one key.

Masked (causal) pairs contribute exactly zero.  [M23] "Exact by Construction"
says the causal ring skips any block strictly in the future of a device's
queries and masks the diagonal block; with positions that is "key position <=
query position" for every pair, and a block with no visible pair is skipped.

Ring order: [RAQA] "The ring" keeps a list kv of the block each device holds
and rotates it with kv = kv[-1:] + kv[:-1] after each round ("pass K/V to the
next device"); [DT2] "Ring Attention" sends to rank+1 and receives from
rank-1.  So at step s device p holds block (p - s) mod N.

Finalize: out = o / l; the log-sum-exp of the visible scaled scores is
m + log l ([DT2] "Vocab-parallel cross-entropy": logsumexp = m + log Z).  A
row that saw nothing has l = 0: out = 0 and lse = -inf.
"""

import numpy as np

from .attention import _as_f64
from .layouts import device_positions


def init_state(rows, d):
    """Running state (m, l, o) for `rows` query rows of head dim d."""
    return (np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, d)))


def absorb_block(state, q, k, v, scale, visible=None):
    """Fold one key/value block into the running state; returns the new state.

    q [r, D]; k, v [n, D]; visible [r, n] bool (None: all pairs visible).

    The block is reduced on its own first: m_b, its row max over the visible
    scores; l_b, the sum of exp(s - m_b); o_b, the sum of exp(s - m_b) v.
    Folding it in is then the recurrence's update written with the block's
    own sums: the running max becomes max(m, m_b), and the old sums and the
    block's are each brought to it (factors exp(m - m') and exp(m_b - m'))
    before they are added.  A block with no visible key for a row adds
    nothing to it; a row that has seen nothing keeps m = -inf, l = 0, o = 0.
    """
    m, l, o = state
    s = (q @ k.T) * scale
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    # the block on its own
    m_b = s.max(axis=1)
    has = np.isfinite(m_b)  # rows that see a key of this block
    e = np.exp(s - np.where(has, m_b, 0.0)[:, None])  # 0 on masked entries
    l_b = np.where(has, e.sum(axis=1), 0.0)
    o_b = np.where(has[:, None], e @ v, 0.0)
    # both sides at the new running max
    m_new = np.maximum(m, m_b)
    ref = np.where(np.isfinite(m_new), m_new, 0.0)
    w_old = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
    w_blk = np.where(has, np.exp(m_b - ref), 0.0)
    return (m_new, l * w_old + l_b * w_blk, o * w_old[:, None] + o_b * w_blk[:, None])


def finalize(state):
    """(out, lse) from a running state."""
    m, l, o = state
    pos = l > 0
    safe_l = np.where(pos, l, 1.0)
    out = np.where(pos[:, None], o / safe_l[:, None], 0.0)
    lse = np.where(pos, m + np.log(safe_l), -np.inf)
    return out, lse


def ring_visit_order(N):
    """Block index that device p holds at step s: order[p][s] = (p - s) mod N."""
    return [[(p - s) % N for s in range(N)] for p in range(N)]


def ring_attention(q, k, v, num_devices, layout="contiguous", causal=False,
                   order=None, scale=None, skip_empty_blocks=True):
    """Simulated ring over `num_devices` devices; inputs and outputs in natural order.

    q [B, Hq, S, D]; k, v [B, Hkv, S, D].  order[p] (optional) is any
    permutation of range(N) giving the blocks device p visits; default is the
    ring order.  Returns (out [B, Hq, S, D], lse [B, Hq, S]) float64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    assert k.shape[2] == S and v.shape[2] == S
    assert Hq % Hkv == 0
    G = Hq // Hkv
    N = num_devices
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if order is None:
        order = ring_visit_order(N)
    pos = [device_positions(S, N, layout, p) for p in range(N)]
    out = np.zeros((B, Hq, S, D))
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for p in range(N):
                qp = pos[p]
                q_blk = q[b, h, qp]
                state = init_state(len(qp), D)
                for j in order[p]:
                    kp = pos[j]
                    vis = (kp[None, :] <= qp[:, None]) if causal else None
                    if vis is not None and skip_empty_blocks and not vis.any():
                        continue
                    state = absorb_block(state, q_blk, k[b, g, kp], v[b, g, kp], scale, vis)
                o, l_ = finalize(state)
                out[b, h, qp] = o
                lse[b, h, qp] = l_
    return out, lse
