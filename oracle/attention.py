"""O1: ordinary (full) softmax attention, written out from its definition.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Definition followed: [M23] "Exact by Construction" builds the single-device
reference as softmax(q k^T * scale) v with scale = 1/sqrt(d), and its causal
reference masks every key strictly after the query (triu(ones, diagonal=1));
[RAQA] "The ring" ends with the same ordinary attention, scores divided by
sqrt(d).  Log-sum-exp is written as m + log Z, as [DT2] "Vocab-parallel
cross-entropy" writes logsumexp(z) = m + log Z.

For each batch b, query head h (key/value head g = h // (Hq/Hkv)) and query
row i:
    visible(i) = { j : k_pos[j] <= q_pos[i] }  if causal, else every key
    s_ij   = (q_i . k_j) * scale                        (fp64)
    M_i    = max_{j in visible(i)} s_ij
    lse_i  = M_i + log( sum_{j in visible(i)} exp(s_ij - M_i) )
    out_i  = sum_{j in visible(i)} exp(s_ij - lse_i) * v_j
A row that sees no key gets out_i = 0 and lse_i = -inf.

Positions are global token positions (whatever the layout), so the causal
rule is "key position <= query position", diagonal included.

Causal rows are computed in chunks, and a chunk only meets the keys whose
position is at most the chunk's last query position: every other key is
masked for every row of the chunk and would add exactly zero ([M23] "Exact by
Construction": the causal ring never computes blocks wholly in a device's
future).  With keys in ascending position order that is a prefix of the key
axis.
"""

import numpy as np


def _as_f64(x):
    """Exact upcast to a float64 numpy array (torch tensors of fp32/bf16 too)."""
    if hasattr(x, "detach"):  # torch tensor; bf16 -> fp32 is exact
        import torch

        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16 or x.dtype == torch.float16:
            x = x.to(torch.float32)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _one_row_block(q_rows, k, v, visible, scale):
    """Rows q_rows [r, D] against keys k, v [Sk, D]; visible [r, Sk] bool or None."""
    if k.shape[0] == 0:  # no key at all: every row is empty
        return np.zeros((q_rows.shape[0], v.shape[1])), np.full(q_rows.shape[0], -np.inf)
    s = (q_rows @ k.T) * scale
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    seen = np.isfinite(m)
    m_safe = np.where(seen, m, 0.0)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 on masked entries
    z = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(seen, m_safe + np.log(np.where(seen, z, 1.0)), -np.inf)
    out = np.where(seen[:, None], (e @ v) / np.where(seen, z, 1.0)[:, None], 0.0)
    return out, lse


def full_attention(q, k, v, q_pos=None, k_pos=None, causal=False, scale=None,
                   row_chunk=256):
    """Full softmax attention.

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D] (any float type; upcast exactly).
    q_pos [Sq], k_pos [Sk]: global token positions (default 0..Sq-1, 0..Sk-1).
    Returns (out [B, Hq, Sq, D] float64, lse [B, Hq, Sq] float64).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0, "query heads must be a multiple of key/value heads"
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    qp = np.arange(Sq) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    kp = np.arange(Sk) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    ascending = bool(np.all(np.diff(kp) >= 0))
    out = np.zeros((B, Hq, Sq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, Sq, row_chunk):
                r1 = min(Sq, r0 + row_chunk)
                kk, vv, vis = k[b, g], v[b, g], None
                if causal:
                    last = qp[r0:r1].max()
                    if ascending:  # the keys any row of the chunk can see: a prefix
                        keys = slice(0, int(np.searchsorted(kp, last, side="right")))
                    else:
                        keys = np.flatnonzero(kp <= last)
                    kk, vv = kk[keys], vv[keys]
                    vis = kp[keys][None, :] <= qp[r0:r1, None]
                o, l_ = _one_row_block(q[b, h, r0:r1], kk, vv, vis, scale)
                out[b, h, r0:r1] = o
                lse[b, h, r0:r1] = l_
    return out, lse


def attention_rows(q, k, v, rows, q_pos=None, k_pos=None, causal=False, scale=None):
    """O1 evaluated only at the listed rows.

    rows: iterable of (b, h, i) with i an index into q's sequence axis.
    Returns (out [n, D] float64, lse [n] float64) in the order given.
    Inputs may be torch tensors or arrays; only the rows' data is upcast,
    with k, v upcast once per (b, g) pair that is needed.
    """
    rows = [tuple(int(t) for t in r) for r in rows]
    Hq = q.shape[1]
    Hkv = k.shape[1]
    D = q.shape[3]
    Sk = k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    kp = np.arange(Sk) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    qp = None if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    out = np.zeros((len(rows), D))
    lse = np.zeros(len(rows))
    by_kv = {}
    for n, (b, h, i) in enumerate(rows):
        by_kv.setdefault((b, h // G), []).append(n)
    for (b, g), idx in by_kv.items():
        kk = _as_f64(k[b, g])
        vv = _as_f64(v[b, g])
        qq = np.stack([_as_f64(q[rows[n][0], rows[n][1], rows[n][2]]) for n in idx])
        vis = None
        if causal:
            pos = np.array([rows[n][2] if qp is None else qp[rows[n][2]] for n in idx])
            vis = kp[None, :] <= pos[:, None]
        o, l_ = _one_row_block(qq, kk, vv, vis, scale)
        out[idx] = o
        lse[idx] = l_
    return out, lse
