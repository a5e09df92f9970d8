"""O1 over many CPU cores: the same full_attention, one task per row range.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

This module adds no arithmetic.  It splits the rows of every (batch, query
head) into ranges, runs oracle.attention.full_attention on each range in a
pool of worker processes (one BLAS thread each, so the number of cores used is
the number of workers), and gathers the results.  Every output row depends on
its own query row and on the keys only, so the split cannot change any value.

Inputs are upcast once to float64 into memory-mapped files (in /dev/shm when
it has room, else in the temporary directory), which the workers map; workers
are started with the "spawn" method, so they hold no GPU state.
"""

import multiprocessing as mp
import os
import shutil
import tempfile
import time
from concurrent.futures import ProcessPoolExecutor, as_completed

import numpy as np

from .attention import _as_f64, full_attention

_W = {}  # worker side: name -> array view of the shared inputs and outputs


MAX_WORKERS = 16  # one GPU's share of a shared host's cores


def default_workers():
    """The cores this process may run on, at most MAX_WORKERS (the pool's default)."""
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _limit_blas():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:
        pass


def _attach(spec):
    _limit_blas()
    for name, (path, shape) in spec.items():
        _W[name] = np.memmap(path, dtype=np.float64, mode="r+", shape=shape)


def _ready(_):
    return os.getpid()


def _task(args):
    b, h, g, r0, r1, causal, scale, row_chunk = args
    q, k, v = _W["q"], _W["k"], _W["v"]
    qp = _W["qpos"][r0:r1].astype(np.int64)
    kp = _W["kpos"].astype(np.int64)
    out, lse = full_attention(q[b, h, r0:r1][None, None], k[b, g][None, None],
                              v[b, g][None, None], q_pos=qp, k_pos=kp, causal=causal,
                              scale=scale, row_chunk=row_chunk)
    _W["out"][b, h, r0:r1] = out[0, 0]
    _W["lse"][b, h, r0:r1] = lse[0, 0]
    return r1 - r0


class _Shared:
    """Named float64 arrays in memory-mapped files of one directory, removed on close()."""

    def __init__(self, nbytes):
        base = None
        if os.path.isdir("/dev/shm"):
            try:
                if shutil.disk_usage("/dev/shm").free > 1.25 * nbytes:
                    base = "/dev/shm"
            except OSError:
                pass
        self.dir = tempfile.mkdtemp(prefix="oracle_pool_", dir=base)
        self.arrays, self.spec = {}, {}

    def add(self, name, shape, init=None):
        path = os.path.join(self.dir, name)
        arr = np.memmap(path, dtype=np.float64, mode="w+", shape=tuple(shape))
        if init is not None:
            arr[...] = init
        self.arrays[name] = arr
        self.spec[name] = (path, tuple(shape))
        return arr

    def close(self):
        self.arrays.clear()
        shutil.rmtree(self.dir, ignore_errors=True)


def _fill_f64(dst, x):
    """dst[...] = x upcast exactly, one leading slice at a time (bounded memory)."""
    for i in range(dst.shape[0]):
        for j in range(dst.shape[1]):
            dst[i, j] = _as_f64(x[i, j])


def full_attention_pool(q, k, v, q_pos=None, k_pos=None, causal=False, scale=None,
                        workers=None, rows_per_task=1024, row_chunk=64, tasks=None,
                        progress=None, progress_every=20.0, time_budget=None,
                        sort_tasks=True):
    """oracle.attention.full_attention, computed by a pool of processes.

    q [B, Hq, Sq, D], k, v [B, Hkv, Sk, D] (torch tensors or arrays, any float
    type); q_pos, k_pos as for full_attention.  tasks: optional list of
    (b, h, r0, r1) row ranges to compute (default: every row); rows outside
    them are left as NaN.  progress(done_rows, total_rows, seconds) is called
    at most every `progress_every` seconds.  time_budget: stop handing out
    tasks once that many seconds have passed (the tasks in flight finish).
    sort_tasks: hand out causal tasks longest first (else in the given order).

    Returns (out [B, Hq, Sq, D], lse [B, Hq, Sq], info) with out and lse
    float64 and info = {"workers", "seconds", "rows", "tasks_done", "cpu_model"};
    seconds counts the pool's work from the first task to the last result, not
    the upcast of the inputs or the start of the workers.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0, "query heads must be a multiple of key/value heads"
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    workers = workers or default_workers()
    qp = np.arange(Sq) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    kp = np.arange(Sk) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    if tasks is None:
        tasks = [(b, h, r0, min(Sq, r0 + rows_per_task))
                 for b in range(B) for h in range(Hq) for r0 in range(0, Sq, rows_per_task)]
    # the longest ranges first (under a causal mask, those with the latest
    # positions), so the pool ends evenly
    if causal and sort_tasks:
        tasks = sorted(tasks, key=lambda t: -int(qp[t[2]:t[3]].max()))
    sh = _Shared(8 * (2 * B * Hq * Sq * D + 2 * B * Hkv * Sk * D + 2 * B * Hq * Sq + Sq + Sk))
    try:
        _fill_f64(sh.add("q", (B, Hq, Sq, D)), q)
        _fill_f64(sh.add("k", (B, Hkv, Sk, D)), k)
        _fill_f64(sh.add("v", (B, Hkv, Sk, D)), v)
        sh.add("qpos", (Sq,), qp)
        sh.add("kpos", (Sk,), kp)
        out = sh.add("out", (B, Hq, Sq, D), np.nan)
        lse = sh.add("lse", (B, Hq, Sq), np.nan)
        total = sum(t[3] - t[2] for t in tasks)
        saved = {n: os.environ.get(n) for n in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                "MKL_NUM_THREADS")}
        os.environ.update({n: "1" for n in saved})  # the workers inherit this at start
        try:
            with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"),
                                     initializer=_attach, initargs=(sh.spec,)) as ex:
                # start every worker before the clock starts
                list(ex.map(_ready, range(workers)))
                t0 = time.perf_counter()
                pending, nxt, done_rows, finished = {}, 0, 0, []
                last = t0

                def submit():
                    nonlocal nxt
                    b, h, r0, r1 = tasks[nxt]
                    f = ex.submit(_task, (b, h, h // G, r0, r1, bool(causal), float(scale),
                                          row_chunk))
                    pending[f] = tasks[nxt]
                    nxt += 1

                while nxt < len(tasks) and len(pending) < 2 * workers:
                    submit()
                while pending:
                    f = next(as_completed(list(pending)))
                    done_rows += f.result()
                    finished.append(pending.pop(f))
                    now = time.perf_counter()
                    in_budget = time_budget is None or now - t0 < time_budget
                    if nxt < len(tasks) and in_budget:
                        submit()
                    if progress is not None and now - last >= progress_every:
                        progress(done_rows, total, now - t0)
                        last = now
                seconds = time.perf_counter() - t0
        finally:
            for n, val in saved.items():
                if val is None:
                    os.environ.pop(n, None)
                else:
                    os.environ[n] = val
        res = (np.array(out), np.array(lse))
    finally:
        sh.close()
    return res[0], res[1], {"workers": workers, "seconds": seconds, "rows": done_rows,
                            "tasks_done": finished, "cpu_model": cpu_model()}
