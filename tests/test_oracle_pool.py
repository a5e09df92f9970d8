"""The process pool that runs O1 over many cores (oracle/parallel.py) adds no
arithmetic: its result equals the serial O1 on every row it computes.  CPU
only; small shapes."""

import numpy as np
import torch

from oracle import attention as O1
from oracle import layouts as OL
from oracle import parallel as OP
from gpu_helpers import rand


def test_pool_equals_serial():
    q = rand((2, 4, 700, 32), 1, torch.float32).to(torch.bfloat16)
    k = rand((2, 2, 700, 32), 2, torch.float32).to(torch.bfloat16)
    v = rand((2, 2, 700, 32), 3, torch.float32).to(torch.bfloat16)
    for causal in (False, True):
        ro, rl = O1.full_attention(q, k, v, causal=causal)
        po, pl, info = OP.full_attention_pool(q, k, v, causal=causal, workers=3,
                                              rows_per_task=128)
        assert info["rows"] == 2 * 4 * 700 and info["workers"] == 3
        assert np.abs(po - ro).max() < 1e-13 and np.abs(pl - rl).max() < 1e-13


def test_pool_device_order_keys_and_subset():
    """Striped device-order keys (positions not ascending) and a task subset:
    rows outside the listed ranges stay NaN, the rest equal the serial O1."""
    S, N = 256, 4
    q = rand((1, 2, S // N, 16), 4, torch.float32)
    k = rand((1, 1, S, 16), 5, torch.float32)
    v = rand((1, 1, S, 16), 6, torch.float32)
    qp = OL.device_positions(S, N, "striped", 1)
    kp = OL.permuted_positions(S, N, "striped")
    ro, rl = O1.full_attention(q, k, v, q_pos=qp, k_pos=kp, causal=True)
    tasks = [(0, 0, 0, 20), (0, 1, 30, 64)]
    po, pl, info = OP.full_attention_pool(q, k, v, q_pos=qp, k_pos=kp, causal=True, workers=2,
                                          tasks=tasks, row_chunk=7)
    assert sorted(info["tasks_done"]) == sorted(tasks) and info["rows"] == 54
    assert np.abs(po[0, 0, :20] - ro[0, 0, :20]).max() < 1e-13
    assert np.abs(pl[0, 1, 30:] - rl[0, 1, 30:]).max() < 1e-13
    assert np.isnan(pl[0, 0, 20:]).all() and np.isnan(pl[0, 1, :30]).all()


def test_pool_time_budget():
    """With a zero budget only the first wave of tasks (two per worker) runs."""
    q = rand((1, 2, 512, 16), 7, torch.float32)
    k = rand((1, 1, 512, 16), 8, torch.float32)
    v = rand((1, 1, 512, 16), 9, torch.float32)
    po, pl, info = OP.full_attention_pool(q, k, v, causal=True, workers=2, rows_per_task=32,
                                          time_budget=0.0)
    assert len(info["tasks_done"]) == 4
    ro, rl = O1.full_attention(q, k, v, causal=True)
    for b, h, r0, r1 in info["tasks_done"]:
        assert np.abs(pl[b, h, r0:r1] - rl[b, h, r0:r1]).max() < 1e-13
