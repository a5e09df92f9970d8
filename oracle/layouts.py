"""Token -> device layouts for the simulated ring, and causal work per device.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Layouts ("device p, local index a" -> global token position), sequence of S
tokens over N devices, blk = S / N tokens per device:
  contiguous  [RAQA] "The ring", step 1: the sequence is cut into N contiguous
              blocks and device i holds block i:      pos = p*blk + a.
  striped     [M23] "The Causal Imbalance -- and the Striped Fix": device p
              holds the interleaved positions p, p+N, p+2N, ...:
                                                       pos = p + a*N.
  zigzag      named on both [M23] (same section) and [RAQA] "The causal-mask
              problem" / "A real-life example" with no formula.  Reading taken:
              cut the sequence into 2N chunks of c = S/(2N); device p holds
              chunk p followed by chunk 2N-1-p, both ascending:
                 a <  c:  pos = p*c + a
                 a >= c:  pos = (2N-1-p)*c + (a - c)
Local indices are ascending in position inside every device's block.

"Device order" is the concatenation of the N device blocks, device 0 first,
so device p's block is the slice [p*blk, (p+1)*blk) of a tensor in device
order.  to_device_order / from_device_order move a tensor between natural
token order and device order along its sequence axis.
"""

import numpy as np

LAYOUTS = ("contiguous", "striped", "zigzag")


def device_positions(S, N, layout, p):
    """Global positions held by device p, in local (ascending) order."""
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    if N < 1 or S % N != 0:
        raise ValueError("the sequence must split into N equal blocks")
    blk = S // N
    a = np.arange(blk, dtype=np.int64)
    if layout == "contiguous":
        return p * blk + a
    if layout == "striped":
        return p + a * N
    if S % (2 * N) != 0:
        raise ValueError("zigzag needs the sequence to split into 2N equal chunks")
    c = S // (2 * N)
    return np.where(a < c, p * c + a, (2 * N - 1 - p) * c + (a - c))


def permuted_positions(S, N, layout):
    """Global position of every index of a device-ordered sequence."""
    return np.concatenate([device_positions(S, N, layout, p) for p in range(N)])


def to_device_order(x, N, layout, axis=-2):
    """Natural token order -> device order along `axis` (a gather)."""
    x = np.asarray(x)
    perm = permuted_positions(x.shape[axis], N, layout)
    return np.take(x, perm, axis=axis)


def from_device_order(y, N, layout, axis=-2):
    """Device order -> natural token order along `axis` (the inverse scatter)."""
    y = np.asarray(y)
    S = y.shape[axis]
    perm = permuted_positions(S, N, layout)
    out = np.empty_like(y)
    idx = [slice(None)] * y.ndim
    idx[axis] = perm
    out[tuple(idx)] = y
    return out


def causal_block_work(num_devices, block_size, layout):
    """Causal (query, key) pairs each device computes, counted pair by pair.

    [M23] "The Causal Imbalance -- and the Striped Fix": a query at position i
    attends to the i+1 keys at positions <= i; the function returns the
    per-device work, max/min imbalance and the total.
    """
    S = num_devices * block_size
    keys = np.arange(S, dtype=np.int64)
    work = []
    for p in range(num_devices):
        qp = device_positions(S, num_devices, layout, p)
        work.append(int((keys[None, :] <= qp[:, None]).sum()))
    return {
        "work": work,
        "imbalance": max(work) / min(work),
        "total": int(sum(work)),
    }
