"""The bench's FLOP counts, checked on the CPU.

bench.py reports algorithmic TFLOP/s: 4 * D FLOPs per visible (query, key)
pair per query head, with the visible pairs in closed form per layout
("Module 23: Distributed Training", "The Causal Imbalance -- and the Striped
Fix"; "Explain ring attention ...", "The causal-mask problem").  Here those
closed forms are compared with a brute-force count over the oracle's layout
maps (every query position against every key position), for the whole ring
and for each device's share.  The executed-pairs model (whole tiles the
matrix-core kernel visits, masked parts included) must cover every visible
pair and equal them where no tile is partly masked."""

import numpy as np
import pytest

import bench
from oracle import layouts as OL


def brute_visible(S, N, layout, causal, device):
    """Visible pairs per query head by enumeration: a query at position qp
    sees key position kp iff kp <= qp (causal), else every key."""
    devs = range(N) if device < 0 else [device]
    kpos = np.arange(S)
    total = 0
    for p in devs:
        qpos = np.asarray(OL.device_positions(S, N, layout, p))
        if causal:
            total += int((kpos[None, :] <= qpos[:, None]).sum())
        else:
            total += qpos.size * S
    return total


CASES = [(S, N) for S, N in ((64, 2), (96, 4), (128, 8), (240, 6))]


@pytest.mark.parametrize("S,N", CASES)
@pytest.mark.parametrize("layout", OL.LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_visible_pairs_closed_forms(S, N, layout, causal):
    if layout == "zigzag" and S % (2 * N):
        pytest.skip("zigzag needs S divisible by 2N")
    for device in [-1] + list(range(N)):
        want = brute_visible(S, N, layout, causal, device)
        got = bench.visible_pairs(S, N, layout, causal, device)
        assert got == want, (S, N, layout, causal, device, got, want)


def test_whole_ring_is_layout_independent():
    """The whole ring sees S(S+1)/2 causal pairs under every layout: a layout
    only moves tokens between devices."""
    S, N = 4096, 8
    for layout in OL.LAYOUTS:
        assert bench.visible_pairs(S, N, layout, True, -1) == S * (S + 1) // 2
        assert brute_visible(S, N, layout, True, -1) == S * (S + 1) // 2


@pytest.mark.parametrize("layout", OL.LAYOUTS)
@pytest.mark.parametrize("G", [1, 4])
def test_executed_pairs_cover_visible(layout, G):
    """Executed pairs >= visible pairs (every visible pair lies in a visited
    tile); non-causal, with blocks a multiple of the tile sizes, they are
    equal (no tile is partly masked)."""
    S, N, D = 8192, 8, 128
    vis = bench.visible_pairs(S, N, layout, True, -1)
    ex = bench.executed_pairs(S, N, layout, True, -1, D, G=G)
    assert ex >= vis
    # the masked excess: in each key block, only the 64-key tiles whose local
    # indices overlap the query tile's (rows / 64 + 1 of them) can be partly
    # visible, each with at most rows x 64 masked pairs
    rows = (8 * 32) >> (2 if G == 4 else 0)
    assert ex - vis <= (S // rows) * N * (rows // 64 + 1) * rows * 64
    assert bench.executed_pairs(S, N, layout, False, -1, D, G=G) == S * S


def test_headline_flops():
    """The 32K-token causal ring: 4 * D * Hq * S(S+1)/2 FLOPs, 8.80 TFLOP."""
    S, Hq, D = 32768, 32, 128
    flops = 4 * D * Hq * bench.visible_pairs(S, 8, "contiguous", True, -1)
    assert flops == 4 * 128 * 32 * (32768 * 32769 // 2)
    assert abs(flops / 1e12 - 8.7964) < 1e-4
