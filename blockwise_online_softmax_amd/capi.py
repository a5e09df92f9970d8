"""ctypes binding of libra.so: the C ABI of include/ra.h, same names.

Argument marshalling only.  Tensors are PyTorch tensors on the GPU; the
binding passes their data pointers and the current HIP stream and raises
RuntimeError with ra_last_error() on a non-OK status.  Every computation
runs in the library's HIP kernels; there is no other path.
"""

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libra.so")

RA_OK = 0
RA_ERR_NULL = 1
RA_ERR_SHAPE = 2
RA_ERR_DTYPE = 3
RA_ERR_ENUM = 4
RA_ERR_UNSUPPORTED = 5
RA_ERR_WORKSPACE = 6
RA_ERR_HIP = 7
STATUS_NAMES = {0: "RA_OK", 1: "RA_ERR_NULL", 2: "RA_ERR_SHAPE", 3: "RA_ERR_DTYPE",
                4: "RA_ERR_ENUM", 5: "RA_ERR_UNSUPPORTED", 6: "RA_ERR_WORKSPACE",
                7: "RA_ERR_HIP"}

RA_F32 = 0
RA_BF16 = 1
RA_MASK_NONE = 0
RA_MASK_CAUSAL = 1
RA_CONTIGUOUS = 0
RA_STRIPED = 1
RA_ZIGZAG = 2
LAYOUT_IDS = {"contiguous": RA_CONTIGUOUS, "striped": RA_STRIPED, "zigzag": RA_ZIGZAG}

EXPORTED = ["ra_state_init", "ra_block_step", "ra_finalize", "ra_ring",
            "ra_ring_workspace_bytes", "ra_permute", "ra_positions", "ra_layout_position",
            "ra_state_merge",
            "ra_merge", "ra_vocab_ce_shard", "ra_vocab_ce_combine", "ra_vocab_ce_grad",
            "ra_vocab_ce_workspace_bytes", "ra_vocab_ce", "ra_vocab_ce_static", "ra_xcd_plan",
            "ra_xcd_speeds", "ra_last_error", "ra_version"]


class RaDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("Sq", ctypes.c_int64), ("Sk", ctypes.c_int64), ("D", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class RaState(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("l", ctypes.c_void_p), ("acc", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Sq", ctypes.c_int64),
                ("D", ctypes.c_int64)]


_lib = None


def load(path=None):
    """Load libra.so (once).  Raises if the library has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    # RA_LIB selects another build of the same library (A/B timing of variants)
    p = path or os.environ.get("RA_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} not found: build the HIP library first "
            "(python -m blockwise_online_softmax_amd.build)")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    dims_p, state_p = ctypes.POINTER(RaDims), ctypes.POINTER(RaState)
    sigs = {
        "ra_state_init": (i32, [state_p, vp]),
        "ra_block_step": (i32, [vp, vp, vp, vp, vp, i32, dims_p, state_p, vp]),
        "ra_finalize": (i32, [state_p, vp, vp, i32, vp]),
        "ra_ring": (i32, [vp, vp, vp, vp, vp, dims_p, i32, i32, i32, i32, vp, sz, vp]),
        "ra_ring_workspace_bytes": (sz, [dims_p, i32, i32, i32]),
        "ra_permute": (i32, [vp, vp, i64, i64, i64, i32, i32, i32, vp]),
        "ra_positions": (i32, [vp, i64, i32, i32, i32, vp]),
        "ra_layout_position": (i64, [i64, i32, i32, i32, i64]),
        "ra_state_merge": (i32, [state_p, state_p, state_p, vp]),
        "ra_merge": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i32, vp]),
        "ra_vocab_ce_shard": (i32, [vp, i64, vp, i64, i64, i64, i32, vp, vp, vp, vp]),
        "ra_vocab_ce_combine": (i32, [vp, vp, vp, i32, i64, vp, vp, vp]),
        "ra_vocab_ce_grad": (i32, [vp, i64, vp, vp, i64, i64, i64, ctypes.c_float, i32, vp, i64,
                                   vp]),
        "ra_vocab_ce_workspace_bytes": (sz, [i64, i32]),
        "ra_vocab_ce": (i32, [vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, sz, vp]),
        "ra_vocab_ce_static": (i32, [vp, vp, i64, i64, i32, i32, vp, vp, vp, vp]),
        "ra_xcd_plan": (i64, [dims_p, i32, i32, i32, i32, vp, vp]),
        "ra_xcd_speeds": (i32, [vp, vp, i32]),
        "ra_last_error": (ctypes.c_char_p, []),
        "ra_version": (i32, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def last_error():
    return load().ra_last_error().decode()


def _check(status, what):
    if status != RA_OK:
        raise RuntimeError(f"{what} failed: {STATUS_NAMES.get(status, status)}: {last_error()}")


# ---------------------------------------------------------------------------
# tensor marshalling


def _torch():
    import torch

    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_id(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def make_dims(q, k, scale=None):
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on batch / head dim")
    return RaDims(B, Hq, Hkv, Sq, Sk, D, _dtype_id(q), 0.0 if scale is None else float(scale))


class State:
    """Caller-owned running state (fp32 m, l, acc) of a query block."""

    def __init__(self, B, Hq, Sq, D, device="cuda"):
        torch = _torch()
        self.m = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device)
        self.l = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device)
        self.acc = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device=device)
        self.shape = (B, Hq, Sq, D)

    def c_struct(self):
        B, Hq, Sq, D = self.shape
        return RaState(self.m.data_ptr(), self.l.data_ptr(), self.acc.data_ptr(), B, Hq, Sq, D)


# ---------------------------------------------------------------------------
# the ABI calls


def ra_state_init(state, stream=None):
    st = state.c_struct()
    _check(load().ra_state_init(ctypes.byref(st), _stream(stream)), "ra_state_init")


def ra_block_step(Q_i, K_j, V_j, q_pos, k_pos, mask_mode, state, scale=None, stream=None):
    for t, n in ((Q_i, "Q_i"), (K_j, "K_j"), (V_j, "V_j")):
        _require(t, n, Q_i.dtype)
    torch = _torch()
    if mask_mode == RA_MASK_CAUSAL:
        _require(q_pos, "q_pos", torch.int32)
        _require(k_pos, "k_pos", torch.int32)
    d = make_dims(Q_i, K_j, scale)
    st = state.c_struct()
    _check(load().ra_block_step(_ptr(Q_i), _ptr(K_j), _ptr(V_j), _ptr(q_pos), _ptr(k_pos),
                                int(mask_mode), ctypes.byref(d), ctypes.byref(st),
                                _stream(stream)), "ra_block_step")


def ra_finalize(state, out, lse=None, stream=None):
    _require(out, "out")
    if lse is not None:
        _require(lse, "lse", _torch().float32)
    st = state.c_struct()
    _check(load().ra_finalize(ctypes.byref(st), _ptr(out), _ptr(lse), _dtype_id(out),
                              _stream(stream)), "ra_finalize")


def ra_ring_workspace_bytes(q, k, N, layout, device=-1, scale=None):
    d = make_dims(q, k, scale)
    n = load().ra_ring_workspace_bytes(ctypes.byref(d), int(N), LAYOUT_IDS.get(layout, layout),
                                       int(device))
    if n == ctypes.c_size_t(-1).value:
        raise RuntimeError(f"ra_ring_workspace_bytes: {last_error()}")
    return int(n)


def ra_ring(Q, K, V, out, lse, N, layout="contiguous", causal=False, device=-1, ws=None,
            scale=None, stream=None):
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (out, "out")):
        _require(t, n, Q.dtype)
    _require(lse, "lse", _torch().float32)
    if ws is not None:
        _require(ws, "ws")
    d = make_dims(Q, K, scale)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().ra_ring(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse), ctypes.byref(d),
                          int(N), LAYOUT_IDS.get(layout, layout), int(bool(causal)), int(device),
                          _ptr(ws), wsb, _stream(stream)), "ra_ring")


def ra_permute(src, dst, N, layout, inverse=False, stream=None):
    """src, dst: [outer, S, ...] tensors; rows are everything after the S axis."""
    _require(src, "src")
    _require(dst, "dst", src.dtype)
    if src.shape != dst.shape:
        raise ValueError("src and dst shapes differ")
    outer = src.shape[0]
    S = src.shape[1]
    row_bytes = src.element_size() * math.prod(src.shape[2:])
    _check(load().ra_permute(_ptr(src), _ptr(dst), outer, S, row_bytes, int(N),
                             LAYOUT_IDS.get(layout, layout), int(bool(inverse)), _stream(stream)),
           "ra_permute")


def ra_positions(pos, S, N, layout, device=-1, stream=None):
    _require(pos, "pos", _torch().int32)
    _check(load().ra_positions(_ptr(pos), int(S), int(N), LAYOUT_IDS.get(layout, layout),
                               int(device), _stream(stream)), "ra_positions")


def ra_xcd_plan(q, k, N, layout, causal, device=-1, speeds=None, scale=None):
    """Split of an ra_ring launch over the 8 XCDs for relative per-XCD speeds
    (host only; default equal).  Returns (grid, M, keep, dbeg, dcnt); grid 0
    means the launch is not split."""
    d = make_dims(q, k, scale)
    sp = (ctypes.c_float * 8)(*([1.0] * 8 if speeds is None else [float(x) for x in speeds]))
    plan = (ctypes.c_int * 25)()
    g = load().ra_xcd_plan(ctypes.byref(d), int(N), LAYOUT_IDS.get(layout, layout),
                           int(bool(causal)), int(device), sp, plan)
    if g < 0:
        raise ValueError(f"ra_xcd_plan: {last_error()}")
    v = list(plan)
    return int(g), v[0], v[1:9], v[9:17], v[17:25]


def ra_xcd_speeds(speeds=None, set=False, measure=False):
    """The current device's per-XCD split.  Default: returns (speeds,
    measurements) of the estimate.  set=True: split ra_ring launches by
    `speeds` from now on, or with speeds=None equally (the library's default,
    which touches no host state).  measure=True: measure the speeds from the
    next launches on (each measured launch copies 192 bytes back on its
    stream)."""
    sp = (ctypes.c_float * 8)(*([1.0] * 8 if speeds is None else [float(x) for x in speeds]))
    n = ctypes.c_int(0)
    mode = 2 if measure else int(bool(set))
    arg = None if (mode == 1 and speeds is None) else sp
    _check(load().ra_xcd_speeds(arg, ctypes.byref(n), mode), "ra_xcd_speeds")
    return list(sp), int(n.value)


def ra_layout_position(S, N, layout, device, index):
    """Global token position of one index (host; the kernels' layout map)."""
    v = load().ra_layout_position(int(S), int(N), LAYOUT_IDS.get(layout, layout), int(device),
                                  int(index))
    if v < 0:
        raise ValueError(f"ra_layout_position: {last_error()}")
    return int(v)


def ra_state_merge(a, b, out, stream=None):
    """out <- merge of states a and b (out may be a or b)."""
    sa, sb, so = a.c_struct(), b.c_struct(), out.c_struct()
    _check(load().ra_state_merge(ctypes.byref(sa), ctypes.byref(sb), ctypes.byref(so),
                                 _stream(stream)), "ra_state_merge")


def ra_merge(out_a, lse_a, out_b, lse_b, out, lse, stream=None):
    """(out, lse) <- merge of two finalized partial results over disjoint key
    sets.  out_*: [..., D] of one dtype; lse_*: [...] fp32.  out / lse may be
    the a or b tensors."""
    for t, n in ((out_a, "out_a"), (out_b, "out_b"), (out, "out")):
        _require(t, n, out_a.dtype)
        if t.shape != out_a.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} differs from {tuple(out_a.shape)}")
    D = out_a.shape[-1]
    rows = out_a.numel() // D if D else 0
    for t, n in ((lse_a, "lse_a"), (lse_b, "lse_b"), (lse, "lse")):
        _require(t, n, _torch().float32)
        if t.numel() != rows:
            raise ValueError(f"{n} has {t.numel()} elements, expected {rows}")
    _check(load().ra_merge(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), _ptr(out),
                           _ptr(lse), rows, D, _dtype_id(out_a), _stream(stream)), "ra_merge")


def _row_stride(t):
    """Row stride (elements) of a 2-D tensor whose rows are dense."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("logits / grad must be 2-D with unit column stride")
    return t.stride(0)


def ra_vocab_ce_shard(logits, target, vocab_start, m, z_sum, pred, stream=None):
    """One vocab shard's row statistics.  logits: [N, V_loc] (a column slice
    of a larger matrix is fine); target: [N] int64 global ids."""
    torch = _torch()
    if not logits.is_cuda:
        raise ValueError("logits must be on the GPU")
    _require(target, "target", torch.int64)
    for t, n in ((m, "m"), (z_sum, "z_sum"), (pred, "pred")):
        _require(t, n, torch.float32)
    N, V_loc = logits.shape
    _check(load().ra_vocab_ce_shard(_ptr(logits), _row_stride(logits), _ptr(target), N, V_loc,
                                    int(vocab_start), _dtype_id(logits), _ptr(m), _ptr(z_sum),
                                    _ptr(pred), _stream(stream)), "ra_vocab_ce_shard")


def ra_vocab_ce_combine(m, z_sum, pred, loss, lse=None, stream=None):
    """Combine [t, N] shard statistics into per-row loss (and lse)."""
    torch = _torch()
    for t, n in ((m, "m"), (z_sum, "z_sum"), (pred, "pred"), (loss, "loss")):
        _require(t, n, torch.float32)
    if lse is not None:
        _require(lse, "lse", torch.float32)
    t, N = m.shape
    _check(load().ra_vocab_ce_combine(_ptr(m), _ptr(z_sum), _ptr(pred), t, N, _ptr(loss),
                                      _ptr(lse), _stream(stream)), "ra_vocab_ce_combine")


def ra_vocab_ce_grad(logits, target, lse, vocab_start, scale, grad, stream=None):
    """grad = scale * (exp(logits - lse) - onehot) for one shard."""
    torch = _torch()
    if not logits.is_cuda or not grad.is_cuda:
        raise ValueError("logits and grad must be on the GPU")
    if grad.dtype != logits.dtype or grad.shape != logits.shape:
        raise ValueError("grad must match the logits' shape and dtype")
    _require(target, "target", torch.int64)
    _require(lse, "lse", torch.float32)
    N, V_loc = logits.shape
    _check(load().ra_vocab_ce_grad(_ptr(logits), _row_stride(logits), _ptr(target), _ptr(lse), N,
                                   V_loc, int(vocab_start), float(scale), _dtype_id(logits),
                                   _ptr(grad), _row_stride(grad), _stream(stream)),
           "ra_vocab_ce_grad")


def ra_vocab_ce_workspace_bytes(N, t):
    n = load().ra_vocab_ce_workspace_bytes(int(N), int(t))
    if n == ctypes.c_size_t(-1).value:
        raise RuntimeError(f"ra_vocab_ce_workspace_bytes: {last_error()}")
    return int(n)


def ra_vocab_ce(logits, target, t, loss, mean_loss, lse=None, ws=None, stream=None):
    """Whole vocab-parallel cross-entropy over t shards of logits [N, V]."""
    torch = _torch()
    _require(logits, "logits")
    _require(target, "target", torch.int64)
    _require(loss, "loss", torch.float32)
    _require(mean_loss, "mean_loss", torch.float32)
    if lse is not None:
        _require(lse, "lse", torch.float32)
    N, V = logits.shape
    if ws is None:
        ws = torch.empty(ra_vocab_ce_workspace_bytes(N, t), dtype=torch.uint8,
                         device=logits.device)
    _check(load().ra_vocab_ce(_ptr(logits), _ptr(target), N, V, int(t), _dtype_id(logits),
                              _ptr(loss), _ptr(mean_loss), _ptr(lse), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "ra_vocab_ce")


def ra_vocab_ce_static(logits, target, t, loss, mean_loss, lse=None, stream=None):
    """ra_vocab_ce with the library's static per-GPU scratch (no workspace)."""
    torch = _torch()
    _require(logits, "logits")
    _require(target, "target", torch.int64)
    _require(loss, "loss", torch.float32)
    _require(mean_loss, "mean_loss", torch.float32)
    if lse is not None:
        _require(lse, "lse", torch.float32)
    N, V = logits.shape
    _check(load().ra_vocab_ce_static(_ptr(logits), _ptr(target), N, V, int(t), _dtype_id(logits),
                                     _ptr(loss), _ptr(mean_loss), _ptr(lse), _stream(stream)),
           "ra_vocab_ce_static")


def ra_version():
    return int(load().ra_version())


# ---------------------------------------------------------------------------
# allocation conveniences (plumbing: torch allocates, the library computes)


def ring_attention(Q, K, V, N, layout="contiguous", causal=False, device=-1, scale=None,
                   stream=None):
    """Allocate out / lse / workspace with torch and call ra_ring."""
    torch = _torch()
    out = torch.empty_like(Q)
    lse = torch.empty(Q.shape[:3], dtype=torch.float32, device=Q.device)
    nws = ra_ring_workspace_bytes(Q, K, N, layout, device, scale)
    ws = torch.empty(nws, dtype=torch.uint8, device=Q.device) if nws > 0 else None
    ra_ring(Q, K, V, out, lse, N, layout, causal, device, ws, scale, stream)
    return out, lse
