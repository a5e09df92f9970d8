"""Pins for the fp64 oracle: facts the pages and the mathematics fix.

Each pin takes the oracle package `o` as its argument (so the mutation test
can run the same pins against copies of the oracle with a planted mistake)
and raises AssertionError when the oracle disagrees with the fact.

Sources (page titles and sections):
  [M23]  "Module 23: Distributed Training": "The Math: One Block at a Time",
         "Exact by Construction", "The Causal Imbalance -- and the Striped Fix".
  [RAQA] "Explain ring attention and how it enables very long contexts across
         multiple devices?": "The ring", "The causal-mask problem".
  [DT2]  "3.6 Distributed Training II ...": "Ring Attention",
         "Vocab-parallel cross-entropy".
  O3 (merge) follows [M23] "The Math" (the fold ignores block order) and
  [DT2] "Vocab-parallel cross-entropy" (max, then sum of rescaled Z); O4
  (vocab-parallel cross-entropy) follows [DT2] "Vocab-parallel
  cross-entropy".
"""

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


def _maxdiff(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d))) if d.size else 0.0


# ---------------------------------------------------------------------------
# [RAQA] "The ring": 4 devices x 3 tokens, d = 8, default_rng(1): the ring
# equals ordinary attention (the page prints True).  Ordinary attention is
# taken from a library softmax here, not from the oracle.
def pin_tiny_ring_equals_ordinary(o):
    from scipy.special import softmax

    from workloads import tiny_inputs

    g = _golden("raqa_tiny_ring.json")
    assert g["printed_allclose_ring_vs_ordinary"] is True
    Q, K, V = tiny_inputs()
    assert Q.shape == (g["N"] * g["blk"], g["d"])
    ref = softmax(Q @ K.T / np.sqrt(g["d"]), axis=1) @ V
    q, k, v = Q[None, None], K[None, None], V[None, None]
    out1, lse1 = o.attention.full_attention(q, k, v)
    out2, lse2 = o.ring.ring_attention(q, k, v, g["N"], "contiguous", causal=False)
    assert _maxdiff(out1[0, 0], ref) < 1e-12
    assert _maxdiff(out2[0, 0], ref) < 1e-12
    assert np.allclose(out2[0, 0], ref)  # the page's own check
    assert _maxdiff(lse1, lse2) < 1e-12


# ---------------------------------------------------------------------------
# O1 against library routines: torch SDPA (fp64, CPU) for out, scipy
# logsumexp for lse; GQA by repeating K/V heads in contiguous groups.
def pin_library_attention(o):
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp

    for (B, Hq, Hkv, Sq, D, causal, seed) in [
        (1, 2, 2, 7, 8, False, 11),
        (2, 4, 2, 19, 16, True, 12),
        (1, 6, 3, 33, 32, True, 13),
        (1, 4, 1, 40, 8, False, 14),
    ]:
        q = _rand((B, Hq, Sq, D), seed)
        k = _rand((B, Hkv, Sq, D), seed + 100)
        v = _rand((B, Hkv, Sq, D), seed + 200)
        out, lse = o.attention.full_attention(q, k, v, causal=causal)
        G = Hq // Hkv
        kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
        vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, is_causal=causal)
        assert _maxdiff(out, ref.numpy()) < 1e-12
        s = np.einsum("bhid,bhjd->bhij", q, kt.numpy()) / np.sqrt(D)
        if causal:
            s = np.where(np.tril(np.ones((Sq, Sq), dtype=bool)), s, -np.inf)
        assert _maxdiff(lse, logsumexp(s, axis=-1)) < 1e-12


# ---------------------------------------------------------------------------
# Brute force on tiny inputs with arbitrary positions: pure-Python loops with
# math.exp over an explicit visible set, including a row that sees no key.
def _brute(q, k, v, qp, kp, causal, scale):
    Sq, D = len(q), len(q[0])
    outs, lses = [], []
    for i in range(Sq):
        vis = [j for j in range(len(k)) if (not causal) or kp[j] <= qp[i]]
        if not vis:
            outs.append([0.0] * D)
            lses.append(-math.inf)
            continue
        sc = {j: sum(q[i][t] * k[j][t] for t in range(D)) * scale for j in vis}
        mx = max(sc.values())
        z = sum(math.exp(sc[j] - mx) for j in vis)
        outs.append([sum(math.exp(sc[j] - mx) * v[j][t] for j in vis) / z for t in range(D)])
        lses.append(mx + math.log(z))
    return np.array(outs), np.array(lses)


def pin_bruteforce(o):
    rng = np.random.default_rng(7)
    D, Sq, Sk = 3, 5, 6
    q = rng.normal(size=(Sq, D))
    k = rng.normal(size=(Sk, D))
    v = rng.normal(size=(Sk, D))
    qp = np.array([4, 0, 9, 2, -1])      # position -1 sees no key
    kp = np.array([3, 0, 8, 1, 5, 2])
    scale = 0.7
    for causal in (False, True):
        bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), qp, kp, causal, scale)
        out, lse = o.attention.full_attention(q[None, None], k[None, None], v[None, None],
                                              q_pos=qp, k_pos=kp, causal=causal, scale=scale)
        assert _maxdiff(out[0, 0], bo) < 1e-12
        assert _maxdiff(lse[0, 0], bl) < 1e-12
        # row chunks of one and two rows, each meeting only the keys it can
        # see (causal pruning), with keys in the given order and sorted by
        # position
        srt = np.argsort(kp, kind="stable")
        for kk, vv, pp in ((k, v, kp), (k[srt], v[srt], kp[srt])):
            for rc in (1, 2):
                out, lse = o.attention.full_attention(q[None, None], kk[None, None],
                                                      vv[None, None], q_pos=qp, k_pos=pp,
                                                      causal=causal, scale=scale, row_chunk=rc)
                assert _maxdiff(out[0, 0], bo) < 1e-12
                assert _maxdiff(lse[0, 0], bl) < 1e-12
        ro, rl = o.attention.attention_rows(q[None, None], k[None, None], v[None, None],
                                            [(0, 0, i) for i in range(Sq)], q_pos=qp,
                                            k_pos=kp, causal=causal, scale=scale)
        assert _maxdiff(ro, bo) < 1e-12 and _maxdiff(rl, bl) < 1e-12
        # the recurrence over two key blocks, then finalize, gives the same
        st = o.ring.init_state(Sq, D)
        for blk in (slice(0, 4), slice(4, 6)):
            vis = (kp[blk][None, :] <= qp[:, None]) if causal else None
            st = o.ring.absorb_block(st, q, k[blk], v[blk], scale, vis)
        fo, fl = o.ring.finalize(st)
        assert _maxdiff(fo, bo) < 1e-12 and _maxdiff(fl, bl) < 1e-12
        # the running max is the largest visible score seen (brute force)
        m = st[0]
        for i in range(Sq):
            vis = [j for j in range(Sk) if (not causal) or kp[j] <= qp[i]]
            want = max((float(q[i] @ k[j]) * scale for j in vis), default=-math.inf)
            assert (m[i] == want) or abs(m[i] - want) < 1e-12


# ---------------------------------------------------------------------------
# N = 1: the ring is one block, i.e. plain softmax attention ([M23] "The Math").
def pin_single_device(o):
    q = _rand((1, 4, 24, 16), 21)
    k = _rand((1, 2, 24, 16), 22)
    v = _rand((1, 2, 24, 16), 23)
    for causal in (False, True):
        a = o.ring.ring_attention(q, k, v, 1, "contiguous", causal=causal)
        b = o.attention.full_attention(q, k, v, causal=causal)
        assert _maxdiff(a[0], b[0]) < 1e-12 and _maxdiff(a[1], b[1]) < 1e-12


# ---------------------------------------------------------------------------
# [M23] "The Math": the fold is order-independent, so any visiting order
# gives ordinary attention.
def pin_order_invariance(o):
    N = 6
    q = _rand((1, 2, 36, 8), 31)
    k = _rand((1, 1, 36, 8), 32)
    v = _rand((1, 1, 36, 8), 33)
    rng = np.random.default_rng(34)
    ref = o.attention.full_attention(q, k, v, causal=True)
    for _ in range(3):
        order = [list(rng.permutation(N)) for _ in range(N)]
        for layout in ("contiguous", "striped", "zigzag"):
            a = o.ring.ring_attention(q, k, v, N, layout, causal=True, order=order)
            assert _maxdiff(a[0], ref[0]) < 1e-12 and _maxdiff(a[1], ref[1]) < 1e-12


# ---------------------------------------------------------------------------
# [M23] "The Causal Imbalance": striping (or zigzag) changes only who holds
# which token, so the causal result in natural order is unchanged.
def pin_layout_invariance(o):
    N = 4
    q = _rand((2, 4, 32, 8), 41)
    k = _rand((2, 2, 32, 8), 42)
    v = _rand((2, 2, 32, 8), 43)
    ref = o.attention.full_attention(q, k, v, causal=True)
    for layout in ("contiguous", "striped", "zigzag"):
        a = o.ring.ring_attention(q, k, v, N, layout, causal=True)
        assert _maxdiff(a[0], ref[0]) < 1e-12 and _maxdiff(a[1], ref[1]) < 1e-12
    for layout in ("contiguous", "striped", "zigzag"):
        a = o.ring.ring_attention(q, k, v, N, layout, causal=False)
        b = o.attention.full_attention(q, k, v, causal=False)
        assert _maxdiff(a[0], b[0]) < 1e-12


# ---------------------------------------------------------------------------
# Closed forms.  Q = 0 makes every score 0: out_i is the mean of the visible
# v_j and lse_i = ln #visible (causal natural order: mean of v_0..v_i,
# ln(i+1)).  Equal keys give the same weights, and lse = s + ln #visible.
def pin_constant_scores(o):
    S, D, N = 24, 8, 4
    v = _rand((1, 1, S, D), 51)
    k = _rand((1, 1, S, D), 52)
    q = np.zeros((1, 1, S, D))
    cum_mean = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    for fn in ("full", "contiguous", "striped", "zigzag"):
        if fn == "full":
            out, lse = o.attention.full_attention(q, k, v, causal=True)
        else:
            out, lse = o.ring.ring_attention(q, k, v, N, fn, causal=True)
        assert _maxdiff(out[0, 0], cum_mean) < 1e-12
        assert _maxdiff(lse[0, 0], np.log(np.arange(1, S + 1))) < 1e-12
    out, lse = o.attention.full_attention(q, k, v, causal=False)
    assert _maxdiff(out[0, 0], np.broadcast_to(v[0, 0].mean(0), (S, D))) < 1e-12
    assert _maxdiff(lse[0, 0], np.full(S, np.log(S))) < 1e-12
    # equal keys: k_j = k for all j
    qq = _rand((1, 1, S, D), 53)
    kk = np.broadcast_to(_rand((1, 1, 1, D), 54), (1, 1, S, D)).copy()
    s_row = (qq[0, 0] @ kk[0, 0, 0]) / np.sqrt(D)
    out, lse = o.ring.ring_attention(qq, kk, v, N, "zigzag", causal=True)
    assert _maxdiff(out[0, 0], cum_mean) < 1e-12
    assert _maxdiff(lse[0, 0], s_row + np.log(np.arange(1, S + 1))) < 1e-12


# ---------------------------------------------------------------------------
# One visible key: the causal row at global position 0 sees only key 0, so
# out = v_0 and lse = s_00 exactly (the diagonal is included, [M23]
# "Exact by Construction": triu(diagonal=1) masks only j > i).
def pin_single_visible_key(o):
    S, D = 16, 8
    q = _rand((1, 1, S, D), 61)
    k = _rand((1, 1, S, D), 62)
    v = _rand((1, 1, S, D), 63)
    s00 = float(q[0, 0, 0] @ k[0, 0, 0]) / np.sqrt(D)
    for layout in ("contiguous", "striped", "zigzag"):
        out, lse = o.ring.ring_attention(q, k, v, 4, layout, causal=True)
        assert _maxdiff(out[0, 0, 0], v[0, 0, 0]) < 1e-15
        assert abs(lse[0, 0, 0] - s00) < 1e-15


# ---------------------------------------------------------------------------
# [M23] "The Causal Imbalance": printed per-device causal pair counts for
# 8 devices x 16 tokens.  Zigzag (derived, not printed): every device holds
# chunks p and 15-p of 8 tokens, 64*15 + 2*36 = 1032 pairs each.  Closed
# forms at a larger size: contiguous device p does b*b*p + b(b+1)/2 and the
# total is S(S+1)/2 for every layout.
def pin_pair_counts(o):
    g = _golden("m23_causal_block_work.json")
    N, b = g["num_devices"], g["block_size"]
    c = o.layouts.causal_block_work(N, b, "contiguous")
    s = o.layouts.causal_block_work(N, b, "striped")
    z = o.layouts.causal_block_work(N, b, "zigzag")
    assert c["work"] == g["contiguous"]["work"]
    assert s["work"] == g["striped"]["work"]
    assert f"{c['imbalance']:.2f}" == g["contiguous"]["imbalance_2dp"]
    assert f"{s['imbalance']:.2f}" == g["striped"]["imbalance_2dp"]
    assert (c["total"] == s["total"]) == g["same_total"]
    assert z["work"] == [1032] * 8 and z["total"] == c["total"]
    N2, b2 = 6, 10
    S2 = N2 * b2
    c2 = o.layouts.causal_block_work(N2, b2, "contiguous")
    assert c2["work"] == [b2 * b2 * p + b2 * (b2 + 1) // 2 for p in range(N2)]
    for lay in ("contiguous", "striped", "zigzag"):
        assert o.layouts.causal_block_work(N2, b2, lay)["total"] == S2 * (S2 + 1) // 2


# ---------------------------------------------------------------------------
# [M23] "Exact by Construction": the fp32 (2, 4, 96, 32) tensors of
# torch.manual_seed(0), 8 devices.  The page's own reference
# (torch.softmax in fp32, causal by masked_fill(triu(1), finfo.min)) agrees
# with the fp64 oracle to its printed tolerance 1e-5, and the fp64 ring
# equals the fp64 full attention.
def pin_m23_fp32_tensors(o):
    import torch

    g = _golden("m23_exact_fp32.json")
    torch.manual_seed(g["torch_manual_seed"])
    q, k, v = (torch.randn(*g["shape_bhsd"]) for _ in range(3))
    scale = 1.0 / q.size(-1) ** 0.5
    ref = torch.softmax(q @ k.transpose(-2, -1) * scale, dim=-1) @ v
    seq = q.size(-2)
    tri = torch.triu(torch.ones(seq, seq, dtype=torch.bool), diagonal=1)
    ref_c = torch.softmax((q @ k.transpose(-2, -1) * scale).masked_fill(
        tri, torch.finfo(q.dtype).min), dim=-1) @ v
    for causal, r in ((False, ref), (True, ref_c)):
        full = o.attention.full_attention(q, k, v, causal=causal)
        ring = o.ring.ring_attention(q, k, v, g["num_devices"], "contiguous", causal=causal)
        assert _maxdiff(full[0], ring[0]) < 1e-12
        assert _maxdiff(full[0], r.double().numpy()) < g["allclose_atol"]


# ---------------------------------------------------------------------------
# Affine invariance of the PV path (the weights of a row sum to one):
# out(V + 1 u^T) = out(V) + u and out(a V) = a out(V); lse does not move.
def pin_affine(o):
    q = _rand((1, 2, 24, 8), 71)
    k = _rand((1, 1, 24, 8), 72)
    v = _rand((1, 1, 24, 8), 73)
    u = _rand((8,), 74)
    a0 = o.ring.ring_attention(q, k, v, 3, "striped", causal=True)
    a1 = o.ring.ring_attention(q, k, v + u, 3, "striped", causal=True)
    a2 = o.ring.ring_attention(q, k, -2.5 * v, 3, "striped", causal=True)
    assert _maxdiff(a1[0], a0[0] + u) < 1e-12
    assert _maxdiff(a2[0], -2.5 * a0[0]) < 1e-12
    assert _maxdiff(a1[1], a0[1]) < 1e-12


# ---------------------------------------------------------------------------
# lse is the log of the normaliser: sum_j exp(s_ij - lse_i) = 1 over the
# visible keys ([DT2] "Vocab-parallel cross-entropy": logsumexp = m + log Z).
def pin_lse_normalises(o):
    S, D = 30, 16
    q = _rand((1, 1, S, D), 81)
    k = _rand((1, 1, S, D), 82)
    v = _rand((1, 1, S, D), 83)
    out, lse = o.ring.ring_attention(q, k, v, 5, "zigzag", causal=True)
    s = q[0, 0] @ k[0, 0].T / np.sqrt(D)
    vis = np.tril(np.ones((S, S), dtype=bool))
    tot = np.where(vis, np.exp(s - lse[0, 0][:, None]), 0.0).sum(axis=1)
    assert _maxdiff(tot, np.ones(S)) < 1e-12


# ---------------------------------------------------------------------------
# Layout maps from their statements: striped device p holds {p, p+N, ...}
# ([M23]); zigzag device p holds chunk p and chunk 2N-1-p of 2N (reading
# taken); contiguous device p holds block p ([RAQA] "The ring").  Device
# order is a permutation and the two reorderings are inverse.
def pin_layout_maps(o):
    S, N = 48, 4
    blk, c = S // N, S // (2 * N)
    for p in range(N):
        assert list(o.layouts.device_positions(S, N, "contiguous", p)) == list(range(p * blk, (p + 1) * blk))
        assert set(o.layouts.device_positions(S, N, "striped", p)) == set(range(p, S, N))
        assert set(o.layouts.device_positions(S, N, "zigzag", p)) == (
            set(range(p * c, (p + 1) * c)) | set(range((2 * N - 1 - p) * c, (2 * N - p) * c)))
        for lay in ("contiguous", "striped", "zigzag"):
            dp = o.layouts.device_positions(S, N, lay, p)
            assert np.all(np.diff(dp) > 0)
    for lay in ("contiguous", "striped", "zigzag"):
        perm = o.layouts.permuted_positions(S, N, lay)
        assert sorted(perm) == list(range(S))
        x = _rand((2, S, 3), 91)
        y = o.layouts.to_device_order(x, N, lay, axis=1)
        for p in range(N):
            dp = o.layouts.device_positions(S, N, lay, p)
            assert np.array_equal(y[:, p * blk:(p + 1) * blk], x[:, dp])
        assert np.array_equal(o.layouts.from_device_order(y, N, lay, axis=1), x)


# ---------------------------------------------------------------------------
# [RAQA] "The ring" rotates the list of held blocks right by one after each
# round (kv = kv[-1:] + kv[:-1]).  Simulating that list gives the block each
# device holds at each step; the oracle's visit order must be the same.
def pin_visit_order(o):
    for N in (1, 2, 4, 7):
        held = list(range(N))
        seen = [[] for _ in range(N)]
        for _ in range(N):
            for dev in range(N):
                seen[dev].append(held[dev])
            held = held[-1:] + held[:-1]
        assert o.ring.ring_visit_order(N) == seen


# ---------------------------------------------------------------------------
# [DT2] "Ring Attention" starts the running max at -1e30 rather than -inf.
# For every row that sees at least one key both starts give the same result;
# the oracle's -inf start must agree with a -1e30 start.
def pin_initial_max_reading(o):
    S, D = 12, 4
    q = _rand((S, D), 101)
    k = _rand((S, D), 102)
    v = _rand((S, D), 103)
    pos = np.arange(S)
    st_inf = o.ring.init_state(S, D)
    st_big = (np.full(S, -1e30), np.zeros(S), np.zeros((S, D)))
    for blk in (slice(8, 12), slice(4, 8), slice(0, 4)):  # reverse ring order
        vis = pos[blk][None, :] <= pos[:, None]
        st_inf = o.ring.absorb_block(st_inf, q, k[blk], v[blk], 0.5, vis)
        st_big = o.ring.absorb_block(st_big, q, k[blk], v[blk], 0.5, vis)
    a = o.ring.finalize(st_inf)
    b = o.ring.finalize(st_big)
    assert _maxdiff(a[0], b[0]) < 1e-12 and _maxdiff(a[1], b[1]) < 1e-12


# ---------------------------------------------------------------------------
# O3 merge: two states over disjoint key sets, merged, equal ordinary
# attention over the union (O1, itself pinned to library routines and brute
# force above).  The key split is random, not contiguous, and positions are
# arbitrary, so with the causal rule some rows see keys on one side only and
# one row (position -1) sees none.
def pin_merge_equals_full(o):
    from scipy.special import logsumexp

    rng = np.random.default_rng(111)
    Sq, Sk, D = 9, 14, 6
    q = rng.normal(size=(Sq, D)) * 1.5
    k = rng.normal(size=(Sk, D)) * 1.5
    v = rng.normal(size=(Sk, D))
    qp = np.array([0, 3, 7, 12, 20, -1, 5, 1, 9])
    kp = rng.permutation(Sk)
    side = rng.permutation(Sk) < 6          # 6 keys on side a, 8 on side b
    side[np.argsort(kp)[0]] = True          # key position 0 on side a
    side[np.argsort(kp)[1]] = False         # key position 1 on side b
    scale = 0.45
    for causal in (False, True):
        parts = []
        for sel in (side, ~side):
            vis = (kp[sel][None, :] <= qp[:, None]) if causal else None
            st = o.ring.absorb_block(o.ring.init_state(Sq, D), q, k[sel], v[sel], scale, vis)
            parts.append(st)
        ref_out, ref_lse = o.attention.full_attention(q[None, None], k[None, None],
                                                      v[None, None], q_pos=qp, k_pos=kp,
                                                      causal=causal, scale=scale)
        ref_out, ref_lse = ref_out[0, 0], ref_lse[0, 0]
        for x, y in ((0, 1), (1, 0)):
            fo, fl = o.ring.finalize(o.merge.merge_states(parts[x], parts[y]))
            assert _maxdiff(fo, ref_out) < 1e-12 and _maxdiff(fl, ref_lse) < 1e-12
            fa, la = o.ring.finalize(parts[x])
            fb, lb = o.ring.finalize(parts[y])
            mo, ml = o.merge.merge_outputs(fa, la, fb, lb)
            assert _maxdiff(mo, ref_out) < 1e-12 and _maxdiff(ml, ref_lse) < 1e-12
            # merged lse is the library log-sum-exp of the two sides' lse
            with np.errstate(divide="ignore"):
                lib = logsumexp(np.stack([la, lb]), axis=0)
            assert _maxdiff(ml, lib) < 1e-12
        if causal:
            assert np.isneginf(ref_lse[5]) and np.all(ref_out[5] == 0)
            # row at position 0 sees only side a, position 1's row sees both
            assert np.isneginf(o.ring.finalize(parts[1])[1][0])


# ---------------------------------------------------------------------------
# O3 merge: special cases.  The empty state (m = -inf, l = 0, o = 0) and the
# empty finalized row (out = 0, lse = -inf) are identities, exactly; two
# empties stay empty; and merging three parts in either grouping agrees.
def pin_merge_identities(o):
    rng = np.random.default_rng(112)
    R, D = 5, 4
    q = rng.normal(size=(R, D))
    k = rng.normal(size=(9, D))
    v = rng.normal(size=(9, D))
    st = o.ring.absorb_block(o.ring.init_state(R, D), q, k[:4], v[:4], 0.5)
    e = o.ring.init_state(R, D)
    for x, y in ((st, e), (e, st)):
        m, l, acc = o.merge.merge_states(x, y)
        assert np.array_equal(m, st[0]) and np.array_equal(l, st[1]) and np.array_equal(acc, st[2])
    m, l, acc = o.merge.merge_states(e, e)
    assert np.all(np.isneginf(m)) and np.all(l == 0) and np.all(acc == 0)
    fo, fl = o.ring.finalize(st)
    zo, zl = np.zeros((R, D)), np.full(R, -np.inf)
    for args in ((fo, fl, zo, zl), (zo, zl, fo, fl)):
        mo, ml = o.merge.merge_outputs(*args)
        assert np.array_equal(mo, fo) and np.array_equal(ml, fl)
    mo, ml = o.merge.merge_outputs(zo, zl, zo, zl)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    # three parts: (a + b) + c == a + (b + c) == ordinary attention
    parts = [o.ring.absorb_block(o.ring.init_state(R, D), q, k[s], v[s], 0.5)
             for s in (slice(0, 3), slice(3, 5), slice(5, 9))]
    left = o.merge.merge_states(o.merge.merge_states(parts[0], parts[1]), parts[2])
    right = o.merge.merge_states(parts[0], o.merge.merge_states(parts[1], parts[2]))
    ref = o.attention.full_attention(q[None, None], k[None, None], v[None, None], scale=0.5)
    for st3 in (left, right):
        fo3, fl3 = o.ring.finalize(st3)
        assert _maxdiff(fo3, ref[0][0, 0]) < 1e-12 and _maxdiff(fl3, ref[1][0, 0]) < 1e-12
    # a dominant side: raising side b's max by 40 makes it the merged max;
    # side a is scaled by exp(m_a - m), not dropped
    sb = (parts[1][0] + 40.0, parts[1][1], parts[1][2])
    mo2 = o.merge.merge_states(parts[0], sb)
    assert np.all(mo2[0] == sb[0])
    assert _maxdiff(mo2[1], sb[1] + parts[0][1] * np.exp(parts[0][0] - sb[0])) < 1e-12


# ---------------------------------------------------------------------------
# O4 vocab-parallel cross-entropy ([DT2] "Vocab-parallel cross-entropy").
# The page's three-step shard algorithm and the plain per-row definition
# against torch's fp64 cross_entropy, for several shard counts, with targets
# on shard boundaries, and the gradient against torch autograd.
def pin_vocab_ce_library(o):
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(121)
    N, V = 37, 48
    z = rng.normal(size=(N, V)) * 3.0
    tg = rng.integers(0, V, size=N)
    tg[:6] = [0, 6, 12, 23, 24, 47]          # first / last columns of shards
    ref = F.cross_entropy(torch.from_numpy(z), torch.from_numpy(tg), reduction="none").numpy()
    assert _maxdiff(o.vocab_ce.cross_entropy_rows(z, tg), ref) < 1e-12
    for t in (1, 2, 4, 8):
        loss, mean, lse = o.vocab_ce.vocab_parallel(z, tg, t)
        assert _maxdiff(loss, ref) < 1e-12, t
        assert abs(mean - ref.mean()) < 1e-12
        from scipy.special import logsumexp
        assert _maxdiff(lse, logsumexp(z, axis=1)) < 1e-12
    # gradient of the mean loss
    zt = torch.from_numpy(z).requires_grad_(True)
    F.cross_entropy(zt, torch.from_numpy(tg)).backward()
    assert _maxdiff(o.vocab_ce.ce_grad(z, tg, 1.0 / N), zt.grad.numpy()) < 1e-12


# O4 closed forms and brute force: uniform logits give log V; a dominant
# target gives ~0; a target outside the vocab gives the bare log-sum-exp; one
# shard's statistics against pure-Python loops with math.exp.
def pin_vocab_ce_closed_forms(o):
    N, V = 4, 24
    z = np.zeros((N, V))
    for t in (1, 3):
        loss, mean, _ = o.vocab_ce.vocab_parallel(z, np.array([0, 5, 23, 11]), t)
        assert _maxdiff(loss, np.full(N, math.log(V))) < 1e-12
    zd = np.zeros((2, V))
    zd[0, 7] = 40.0
    zd[1, 7] = 40.0
    loss, _, _ = o.vocab_ce.vocab_parallel(zd, np.array([7, 8]), 4)
    assert abs(loss[0] - math.log1p((V - 1) * math.exp(-40.0))) < 1e-15
    assert abs(loss[1] - (40.0 + math.log1p((V - 1) * math.exp(-40.0)))) < 1e-12
    rng = np.random.default_rng(122)
    zr = rng.normal(size=(3, V))
    loss, _, lse = o.vocab_ce.vocab_parallel(zr, np.array([-1, V, 2]), 2)
    assert abs(loss[0] - lse[0]) < 1e-15 and abs(loss[1] - lse[1]) < 1e-15
    assert abs(loss[2] - (lse[2] - zr[2, 2])) < 1e-12
    # one shard, brute force
    start, V_loc = 8, 8
    tg = np.array([9, 3, 15])
    m, s, pred = o.vocab_ce.shard_stats(zr[:, start:start + V_loc], tg, start)
    for r in range(3):
        row = [float(x) for x in zr[r, start:start + V_loc]]
        mx = max(row)
        assert m[r] == mx
        assert abs(s[r] - sum(math.exp(x - mx) for x in row)) < 1e-12
        want = row[tg[r] - start] if start <= tg[r] < start + V_loc else 0.0
        assert pred[r] == want
    # gradient rows sum to zero; the target entry is softmax - 1
    g = o.vocab_ce.ce_grad(zr, np.array([0, 5, 2]), 1.0)
    assert _maxdiff(g.sum(axis=1), np.zeros(3)) < 1e-12
    from scipy.special import softmax
    assert abs(g[1, 5] - (softmax(zr[1])[5] - 1.0)) < 1e-12


ALL_PINS = [
    pin_tiny_ring_equals_ordinary,
    pin_library_attention,
    pin_bruteforce,
    pin_single_device,
    pin_order_invariance,
    pin_layout_invariance,
    pin_constant_scores,
    pin_single_visible_key,
    pin_pair_counts,
    pin_m23_fp32_tensors,
    pin_affine,
    pin_lse_normalises,
    pin_layout_maps,
    pin_visit_order,
    pin_initial_max_reading,
    pin_merge_equals_full,
    pin_merge_identities,
    pin_vocab_ce_library,
    pin_vocab_ce_closed_forms,
]
