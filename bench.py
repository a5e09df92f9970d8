"""Ring-attention throughput on one MI355X, against the bf16 matrix-core roofline.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one ra_ring call: the whole simulated ring (all N virtual devices)
over one batch of seeded synthetic input already resident in HBM.  The
default workload is the Llama-3-8B-shaped causal ring: S = 32768 tokens over
N = 8 virtual devices (blocks of 4096), 32 query / 8 key-value heads, head
dim 128, bf16, contiguous layout.

FLOPs are algorithmic: 4 * D per visible (query, key) pair per query head
(2D for q.k, 2D for p.v), causal pairs counted exactly.  The printed JSON line
carries value = TFLOP/s, the roofline object for the attention kernel (timed
with HIP events on the stream it runs on) and the oracle's CPU rate on a
bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)

WORKLOADS = {
    # name: (workload key in workloads.py, layout, device)
    "gqa32k": ("gqa32k", "contiguous", -1),
    "mha16k": ("mha16k", "contiguous", -1),
    "gqa64k-contiguous": ("gqa64k", "contiguous", -1),
    "gqa64k-striped": ("gqa64k", "striped", -1),
    "gqa64k-zigzag": ("gqa64k", "zigzag", -1),
    "share1m": ("share1m", "zigzag", 0),
}


def visible_pairs(S, N, layout, causal, device):
    """Exact visible (query, key) pairs per query head (closed forms).

    Whole ring: S^2 non-causal, S(S+1)/2 causal (every layout).  Device
    share under zigzag causal: chunks c = S/2N; device p holds chunk p
    (positions p*c + a, each sees p*c + a + 1 keys) and chunk 2N-1-p.
    """
    if device < 0:
        return S * S if not causal else S * (S + 1) // 2
    blk = S // N
    if not causal:
        return blk * S
    if layout == "zigzag":
        c = S // (2 * N)
        first = sum_range(device * c + 1, device * c + c)
        second = sum_range((2 * N - 1 - device) * c + 1, (2 * N - device) * c)
        return first + second
    if layout == "contiguous":
        return sum_range(device * blk + 1, device * blk + blk)
    return sum(device + a * N + 1 for a in range(blk))


def sum_range(lo, hi):
    return (lo + hi) * (hi - lo + 1) // 2


def layout_pos(layout, N, blk, dev, a):
    """Global position of local index a (array) on device dev."""
    a = np.asarray(a, dtype=np.int64)
    if layout == "striped":
        return dev + a * N
    if layout == "zigzag":
        c = blk // 2
        return np.where(a < c, dev * c + a, (2 * N - 1 - dev) * c + (a - c))
    return dev * blk + a


def executed_pairs(S, N, layout, causal, device, D, G=1, tile_keys=64):
    """(query, key) pairs the matrix-core ring kernel computes per query head,
    masked ones included: every (query tile, key tile) it visits in full.  A
    workgroup has 8 wavefronts (D = 128 and blocks of >= 256 rows) or 4, of 32
    rows each, spread over 2^gpl query heads of one kv head (the largest power
    of two dividing G = Hq / Hkv, at most the wavefront count) on the same
    positions, so a query tile is 32 x waves / 2^gpl positions; key tiles are
    64 keys.  Positions ascend inside a device block, so under the causal
    mask a key block is skipped when its first key follows the tile's last
    query, and otherwise runs up to its last tile that starts at or before
    that query.  The excess over the visible pairs is the work done on masked
    parts of diagonal tiles."""
    blk = S // N
    nw = 8 if (D == 128 and blk >= 256) else 4
    gpl = 0
    while (2 << gpl) <= nw and G % (2 << gpl) == 0:
        gpl += 1
    rows = (nw * 32) >> gpl
    devs = range(N) if device < 0 else [device]
    ntile = -(-blk // tile_keys)
    tile_first = np.arange(ntile) * tile_keys
    total = 0
    for p in devs:
        for a0 in range(0, blk, rows):
            nr = min(rows, blk - a0)
            qmax = int(layout_pos(layout, N, blk, p, a0 + nr - 1)) if causal else None
            for j in range(N):
                if not causal:
                    n = ntile
                else:
                    firsts = layout_pos(layout, N, blk, j, tile_first)
                    n = int((firsts <= qmax).sum())
                total += nr * n * tile_keys
    return total


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa32k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target oracle time for the CPU baseline sample")
    ap.add_argument("--step-sweep", action="store_true",
                    help="state-in-HBM ra_block_step on the 32K-token, 32/8-head query set cut "
                         "into blocks of 128..1024 tokens (HBM GB/s); one JSON line per block size")
    ap.add_argument("--layout-balance", action="store_true",
                    help="the 64K causal case per layout: whole ring, permute / un-permute GB/s, "
                         "each virtual device's share and the simulated ring makespan")
    ap.add_argument("--tiny", action="store_true",
                    help="the pages' 4 x 3 tokens x d=8 case: microseconds per ra_ring call")
    ap.add_argument("--merge", action="store_true",
                    help="ra_merge and ra_state_merge on the rows of the 32K-token x 32-head "
                         "x D=128 query set (HBM GB/s); one JSON line each")
    ap.add_argument("--vocab-ce", action="store_true",
                    help="vocab-parallel cross-entropy forward and gradient on 8192 rows x 128,256 "
                         "bf16 logits over 8 shards (HBM GB/s); one JSON line each")
    ap.add_argument("--xcd", choices=("measured", "equal"), default="measured",
                    help="split of the ring launch over the 8 XCDs: by speeds measured during "
                         "the warm-up and then frozen (default), or equal")
    ap.add_argument("--xcd-ab", action="store_true",
                    help="the --workload ring with the even split over the 8 XCDs against the split "
                         "sized by the measured XCD speeds (both frozen), alternating; one JSON line")
    ap.add_argument("--tile-mix", action="store_true",
                    help="timing probe of the attention tile loop's instruction mix (MFMA, LDS "
                         "operand reads, softmax) without copies or barriers, beside the gqa32k "
                         "ring; one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (contiguous ra_permute) so that "
                         "HBM byte counters can be scaled against a kernel of known traffic")
    return ap.parse_args()


def tile_mix(args):
    """The attention tile loop's instruction mix in isolation (libra_probe.so,
    tile_mix_kernel): one workgroup per CU issuing v_mfma_f32_32x32x16_bf16 on
    data-like bf16 operands, with or without the LDS operand reads and the
    softmax work of the ring kernel, in launches of ~35 ms so that the clock
    settles; the five configurations run in rotating rounds.  Beside it, the
    gqa32k ring (even XCD split) in the same units: MFMAs issued per
    microsecond per CU (executed FLOPs / 32768)."""
    import ctypes

    import torch

    import blockwise_online_softmax_amd as ra
    import workloads

    lib = ctypes.CDLL(os.path.join(HERE, "blockwise_online_softmax_amd", "libra_probe.so"))
    fn = lib.ra_probe_tile_mix
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                   ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_longlong),
                   ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    names = ["mfma only (8 waves)", "mfma + softmax (8 waves)",
             "mfma + 1 KB LDS per MFMA (8 waves)",
             "mfma + 1 KB LDS per MFMA + softmax (8 waves: the ring kernel's mix)",
             "mfma + 0.5 KB LDS per MFMA + softmax (4 waves of 64 query rows)"]
    iters = 110000

    def run(cfg):
        ms, n = ctypes.c_float(), ctypes.c_longlong()
        rc = fn(cfg, cus, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(ms),
                ctypes.byref(n), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"ra_probe_tile_mix failed with HIP error {rc}")
        return n.value / (ms.value * 1e3)

    for cfg in range(len(names)):  # warm-up
        run(cfg)
    rates = {c: [] for c in range(len(names))}
    for r in range(3):
        for i in range(len(names)):
            cfg = (i + r) % len(names)
            rates[cfg].append(run(cfg))
    # the gqa32k ring in the same units
    wkey, layout, device = WORKLOADS["gqa32k"]
    cfgw = workloads.WORKLOADS[wkey]
    q, k, v = (t.cuda() for t in workloads.workload_inputs(wkey))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    ms = timed(lambda: ra.ra_ring(q, k, v, out, lse, cfgw["N"], layout, True, -1, None,
                                  stream=stream), 10, 5, stream, min_warm_s=0.5)
    exec_flops = 4.0 * cfgw["D"] * cfgw["Hq"] * executed_pairs(
        cfgw["S"], cfgw["N"], layout, True, -1, cfgw["D"], G=cfgw["Hq"] // cfgw["Hkv"])
    ring_rate = exec_flops / 32768.0 / cus / (ms * 1e3)
    res = {names[c]: round(float(np.median(v)), 1) for c, v in rates.items()}
    print(json.dumps({"metric": "MFMAs per microsecond per CU (tile-loop mix probe)",
                      "probe": res, "gqa32k_ring": round(ring_rate, 1),
                      "gqa32k_ring_ms": round(ms, 3),
                      "ring_over_its_mix": round(ring_rate / res[names[3]], 3),
                      "launches_per_config": 3, "iters": iters, "cus": cus}), flush=True)


def copy_calibration():
    """One contiguous-layout ra_permute over 1 GiB: reads 1 GiB and writes 1 GiB."""
    import torch

    import blockwise_online_softmax_amd as ra

    n = 1 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    rows = src.view(1, n // 256, 64)
    for _ in range(3):
        ra.ra_permute(rows, dst.view(1, n // 256, 64), 1, "contiguous")
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}), flush=True)


def mfma_ceiling():
    """The sustained bf16 matrix-core rate of this GPU and its shader clock
    under that load, from libra_probe.so: 4 workgroups of 512 threads per CU,
    every wavefront issuing 4 independent v_mfma_f32_32x32x16_bf16 chains, on
    operands that look like N(0,1) bf16 data (the clock under MFMA load
    depends on how many operand bits toggle) and, for reference, on small
    constants.  The clock is the shader-clock counter over the constant-rate
    counter of each workgroup's first wavefront (median over workgroups)."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(HERE, "blockwise_online_softmax_amd", "libra_probe.so"))
    fn = lib.ra_probe_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = 4 * cus, 16384  # ~7 ms per launch: long enough for the clock to settle
    sink = torch.empty(wgs * 512, dtype=torch.float32, device="cuda")
    clk = torch.empty(2 * wgs, dtype=torch.int64, device="cuda")
    ms, khz = ctypes.c_float(), ctypes.c_int()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flops = wgs * 8 * iters * 4 * 32768.0
    res = {}
    for random, key in ((1, "random_operands"), (0, "constant_operands")):
        best = None
        for _ in range(3):
            rc = fn(wgs, iters, random, ctypes.c_void_p(sink.data_ptr()),
                    ctypes.c_void_p(clk.data_ptr()), ctypes.byref(ms), ctypes.byref(khz), stream)
            if rc != 0:
                raise RuntimeError(f"ra_probe_mfma failed with HIP error {rc}")
            best = ms.value if best is None else min(best, ms.value)
        c = clk.cpu().numpy().reshape(-1, 2).astype(np.float64)
        mhz = float(np.median(c[:, 0] / c[:, 1])) * khz.value / 1e3
        res[key] = {"tflops": round(flops / (best * 1e-3) / 1e12, 1), "sclk_mhz": round(mhz, 0)}
    out = dict(res["random_operands"])
    out["spec_tflops_at_that_clock"] = round(cus * 4 * 1024 * out["sclk_mhz"] * 1e6 / 1e12, 1)
    out["constant_operands"] = res["constant_operands"]
    out.update({"workgroups": wgs, "mfma_per_wave": iters * 4})
    return out


KERNEL_SOURCES = ["blockwise_online_softmax_amd/csrc/ra_attn_mfma.hip",
                  "blockwise_online_softmax_amd/csrc/ra_internal.h"]


def kernel_sources_sha256():
    """sha256 over the attention kernel's source files, in KERNEL_SOURCES order."""
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch of the attention kernel from the committed counter
    record (profiles/attn_mfma_<workload>_traffic.json), or None when there is
    no record or the kernel's sources changed since the counters were taken."""
    path = os.path.join(HERE, "profiles", f"attn_mfma_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources") != KERNEL_SOURCES or \
            rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    return int(rec["hbm_bytes_per_launch"])


def cpu_baseline(q, k, v, cfg, layout, device, seconds, gpu_out=None, gpu_lse=None):
    """The oracle (O1, fp64 numpy) on a bounded seeded sample of the same
    workload, run by its process pool: one worker per allowed core (at most
    16), one BLAS thread each, causal rows meeting only the keys they can
    see.  Tasks are 64-row ranges of (head, rows) drawn in a seeded random
    order, handed out until `seconds` have passed.  The rate is the
    algorithmic FLOPs of the rows done over the pool's time (the upcast of the
    inputs and the start of the workers are not counted); the time of the
    whole workload is extrapolated from it."""
    from oracle import layouts as OL
    from oracle import parallel as OP

    S, N, D, Hq = cfg["S"], cfg["N"], cfg["D"], cfg["Hq"]
    Sq = q.shape[2]
    causal = cfg["causal"]
    if device >= 0:
        # keys in natural order (the oracle works on positions, so reordering
        # keys together with their positions changes nothing)
        qpos = OL.device_positions(S, N, layout, device)
        kpos = OL.permuted_positions(S, N, layout)
        order = np.argsort(kpos, kind="stable")
        k, v, kpos = k[:, :, order], v[:, :, order], kpos[order]
    else:
        qpos, kpos = np.arange(S), np.arange(S)
    rows_per_task = 64
    tasks = [(0, h, r0, min(Sq, r0 + rows_per_task)) for h in range(Hq)
             for r0 in range(0, Sq, rows_per_task)]
    rng = np.random.default_rng(1000)
    tasks = [tasks[i] for i in rng.permutation(len(tasks))]
    out, lse, info = OP.full_attention_pool(q, k, v, q_pos=qpos, k_pos=kpos, causal=causal,
                                            tasks=tasks, sort_tasks=False, time_budget=seconds)
    kp_sorted = np.sort(kpos)

    def row_pairs(r0, r1):  # visible keys of rows r0..r1-1, summed
        if not causal:
            return (r1 - r0) * len(kpos)
        return int(np.searchsorted(kp_sorted, qpos[r0:r1], side="right").sum())

    pairs = sum(row_pairs(r0, r1) for _, _, r0, r1 in info["tasks_done"])
    all_pairs = Hq * row_pairs(0, Sq)
    errs = [0.0, 0.0]
    if gpu_out is not None:
        for _, h, r0, r1 in info["tasks_done"]:
            go = gpu_out[0, h, r0:r1].float().numpy()
            errs[0] = max(errs[0], float(np.abs(go - out[0, h, r0:r1]).max()))
            errs[1] = max(errs[1], float(np.abs(gpu_lse[0, h, r0:r1].numpy() - lse[0, h, r0:r1]).max()))
    rate = pairs / info["seconds"]
    flops = 4.0 * D * pairs
    return {
        "value": flops / info["seconds"] / 1e12,
        "unit": "TFLOP/s",
        "cores": info["workers"],
        "kind": "oracle",
        "sample": f"{info['rows']} of {Hq * Sq} (head, row) outputs of the same workload "
                  f"({len(info['tasks_done'])} seeded 64-row ranges), fp64 numpy O1, "
                  f"{info['workers']} worker processes x 1 BLAS thread, {info['seconds']:.1f} s, "
                  f"{pairs} visible pairs",
        "cpu_model": info["cpu_model"],
        "pool_seconds": round(info["seconds"], 2),
        "full_workload_seconds_extrapolated": round(all_pairs / rate, 1),
    }, errs


def ms_stats(ms):
    """Mean, median and minimum of per-launch times in ms."""
    return {"mean": round(float(np.mean(ms)), 4), "median": round(float(np.median(ms)), 4),
            "min": round(float(np.min(ms)), 4), "n": len(ms)}


def timed(fn, steps, warmup, stream, min_warm_s=0.1, stats=False):
    """Mean ms of fn() over `steps` launches, HIP events on `stream` (with
    stats=True: the mean, median and minimum).  The warm-up runs `warmup`
    calls and then keeps calling until `min_warm_s` seconds have passed: the
    shader clock ramps over the first tens of milliseconds of load, longer than
    a few calls of a sub-millisecond kernel take."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        fn()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    return ms_stats(ms) if stats else float(np.mean(ms))


def step_sweep(args):
    """ra_block_step with the state in HBM (fp32 m, l, acc read and written
    per step), non-causal, on the 32768-token x 32/8-head x D=128 query set cut
    into `batch` = 32768/blk independent blocks of blk tokens, each folding one
    key/value block of blk tokens.  Bytes per step are algorithmic: Q read,
    K and V read, acc/m/l read and written."""
    import torch

    import blockwise_online_softmax_amd as ra

    Hq, Hkv, D, total = 32, 8, 128, 32768
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda")
    for blk in (128, 256, 512, 1024):
        g.manual_seed(blk)
        batch = total // blk
        q = torch.randn((batch, Hq, blk, D), generator=g, device="cuda").to(torch.bfloat16)
        k = torch.randn((batch, Hkv, blk, D), generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn((batch, Hkv, blk, D), generator=g, device="cuda").to(torch.bfloat16)
        st = ra.State(batch, Hq, blk, D)
        ra.ra_state_init(st)

        def step():
            ra.ra_block_step(q, k, v, None, None, ra.RA_MASK_NONE, st, stream=stream)

        ms = timed(step, args.steps, args.warmup, stream)
        nbytes = batch * blk * (Hq * (2 * D + 8 * D + 16) + Hkv * 2 * 2 * D)
        flops = 4.0 * D * Hq * batch * blk * blk
        gbs = nbytes / (ms * 1e-3) / 1e9
        print(json.dumps({
            "metric": "ra_block_step HBM GB/s (state in HBM, small blocks)", "block_tokens": blk,
            "batch": batch, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "dtype": "bf16",
            "us_per_step": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
            "gb_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "tflop_per_s": round(flops / (ms * 1e-3) / 1e12, 1),
            "flop_per_byte": round(flops / nbytes, 1), "steps": args.steps, "data": "synthetic"}),
            flush=True)
        del q, k, v, st
        torch.cuda.empty_cache()


def interleaved_whole_rings(qd, kd, vd, out, lse, N, layouts, args, stream):
    """Whole causal rings of every layout on the same tensors, timed in
    interleaved rounds (the layout order rotates from round to round) after a
    common warm-up, so that the clock's drift over the run falls on every
    layout alike.  Per layout: mean, median and minimum over all its timed
    launches (HIP events on the launch stream)."""
    import torch

    import blockwise_online_softmax_amd as ra

    calls = {}
    for layout in layouts:
        nws = ra.ra_ring_workspace_bytes(qd, kd, N, layout, -1)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
        calls[layout] = (lambda L=layout, W=ws: ra.ra_ring(qd, kd, vd, out, lse, N, L, True, -1, W,
                                                          stream=stream))
    for layout in layouts:  # warm-up: every layout, then until 0.5 s have passed
        for _ in range(args.warmup):
            calls[layout]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:
        for layout in layouts:
            calls[layout]()
        torch.cuda.synchronize()
    rounds, per = max(3, args.steps), 2
    ms = {layout: [] for layout in layouts}
    for r in range(rounds):
        order = layouts[r % len(layouts):] + layouts[:r % len(layouts)]
        for layout in order:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(per)]
            for a, b in ev:
                a.record(stream)
                calls[layout]()
                b.record(stream)
            torch.cuda.synchronize()
            ms[layout] += [a.elapsed_time(b) for a, b in ev]
    return {layout: ms_stats(v) for layout, v in ms.items()}


def layout_balance(args):
    """The 64K-token causal ring (32/8 heads, D=128, N=8) under each layout:
    the whole ring on one GPU (device = -1; the three layouts timed in
    interleaved rounds on the same tensors),
    the permute and un-permute passes alone, and each virtual device's share
    (device = p) whose maximum is the makespan of an N-GPU ring that overlaps
    its key/value passes."""
    import torch

    import blockwise_online_softmax_amd as ra
    import workloads

    cfg = workloads.WORKLOADS["gqa64k"]
    S, N, D, Hq, Hkv = cfg["S"], cfg["N"], cfg["D"], cfg["Hq"], cfg["Hkv"]
    blk = S // N
    print("# generating inputs for gqa64k", file=sys.stderr, flush=True)
    q, k, v = workloads.workload_inputs("gqa64k")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    del q, k, v
    stream = torch.cuda.current_stream()
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    layouts = ("contiguous", "striped", "zigzag")
    whole = interleaved_whole_rings(qd, kd, vd, out, lse, N, layouts, args, stream)
    for layout in layouts:
        st_whole = whole[layout]
        t_whole = st_whole["mean"]
        rec = {"metric": "causal ring layout balance (64K tokens, N=8)", "layout": layout,
               "whole_ring_ms": round(t_whole, 3), "whole_ring_ms_median": st_whole["median"],
               "whole_ring_ms_min": st_whole["min"]}
        # device-order copies of Q, K, V (the shares' inputs); permute / un-permute timing
        qp, kp, vp = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        if layout != "contiguous":
            def fwd():
                ra.ra_permute(qd.view(Hq, S, D), qp.view(Hq, S, D), N, layout, stream=stream)
                ra.ra_permute(kd.view(Hkv, S, D), kp.view(Hkv, S, D), N, layout, stream=stream)
                ra.ra_permute(vd.view(Hkv, S, D), vp.view(Hkv, S, D), N, layout, stream=stream)

            t_f = timed(fwd, args.steps, args.warmup, stream)
            fbytes = 2 * 2 * S * D * (Hq + 2 * Hkv)
            inv_out = torch.empty_like(qd)
            lse2 = torch.empty_like(lse)

            def inv():
                ra.ra_permute(qp.view(Hq, S, D), inv_out.view(Hq, S, D), N, layout, inverse=True,
                              stream=stream)
                ra.ra_permute(lse.view(Hq, S, 1), lse2.view(Hq, S, 1), N, layout, inverse=True,
                              stream=stream)
            t_i = timed(inv, args.steps, args.warmup, stream)
            ibytes = 2 * (2 * S * D * Hq + 4 * S * Hq)
            rec.update({"permute_ms": round(t_f, 3), "permute_gb_per_s": round(fbytes / (t_f * 1e-3) / 1e9, 1),
                        "unpermute_ms": round(t_i, 3),
                        "unpermute_gb_per_s": round(ibytes / (t_i * 1e-3) / 1e9, 1)})
        else:
            qp.copy_(qd), kp.copy_(kd), vp.copy_(vd)
        dev_ms = []
        oshare = torch.empty((1, Hq, blk, D), dtype=qd.dtype, device="cuda")
        lshare = torch.empty((1, Hq, blk), dtype=torch.float32, device="cuda")
        for p in range(N):
            qs = qp[:, :, p * blk:(p + 1) * blk].contiguous()
            t = timed(lambda: ra.ra_ring(qs, kp, vp, oshare, lshare, N, layout, True, p, None,
                                         stream=stream), max(2, args.steps // 2), 2, stream)
            dev_ms.append(round(t, 3))
        mk = max(dev_ms)
        rec.update({"device_share_ms": dev_ms, "makespan_ms": mk,
                    "imbalance_max_over_mean": round(mk / float(np.mean(dev_ms)), 3),
                    "tokens_per_s_one_gpu": round(S / (t_whole * 1e-3), 1),
                    "tokens_per_s_projected_ring": round(S / (mk * 1e-3), 1)})
        print(json.dumps(rec), flush=True)
        del qp, kp, vp
        torch.cuda.empty_cache()


def merge_bench(args):
    """ra_merge (bf16 out + fp32 lse) and ra_state_merge (fp32 m, l, acc) on
    the rows of a 32768-token x 32-head x D=128 query set, two partial
    results merged into a third buffer.  Bytes are algorithmic: both inputs
    read once, the output written once."""
    import torch

    import blockwise_online_softmax_amd as ra

    B, Hq, S, D = 1, 32, 32768, 128
    rows = B * Hq * S
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    oa = torch.randn((B, Hq, S, D), generator=g, device="cuda").to(torch.bfloat16)
    ob = torch.randn((B, Hq, S, D), generator=g, device="cuda").to(torch.bfloat16)
    la = torch.randn((B, Hq, S), generator=g, device="cuda") * 4
    lb = torch.randn((B, Hq, S), generator=g, device="cuda") * 4
    oo, lo = torch.empty_like(oa), torch.empty_like(la)
    ms = timed(lambda: ra.ra_merge(oa, la, ob, lb, oo, lo, stream=stream), args.steps,
               args.warmup, stream)
    nbytes = rows * 3 * (D * 2 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "ra_merge HBM GB/s (bf16 out, fp32 lse)", "rows": rows, "head_dim": D,
        "us_per_call": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
        "gb_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "steps": args.steps, "data": "synthetic"}), flush=True)
    del oa, ob, oo, la, lb, lo
    st = [ra.State(B, Hq, S, D) for _ in range(3)]
    for i, x in enumerate(st[:2]):
        x.m.normal_(generator=g).mul_(4)
        x.l.uniform_(1, 100, generator=g)
        x.acc.normal_(generator=g)
    ms = timed(lambda: ra.ra_state_merge(st[0], st[1], st[2], stream=stream), args.steps,
               args.warmup, stream)
    nbytes = rows * 3 * (D * 4 + 8)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "ra_state_merge HBM GB/s (fp32 m, l, acc)", "rows": rows, "head_dim": D,
        "us_per_call": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
        "gb_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "steps": args.steps, "data": "synthetic"}), flush=True)


def vocab_ce_bench(args):
    """Vocab-parallel cross-entropy on 8192 rows of bf16 logits over a
    128,256-entry vocabulary (Llama-3's) split into 8 shards: the forward
    (shard statistics + combine + mean) and the gradient of the mean loss.
    Bytes are algorithmic: the forward reads the logits once (plus targets
    and the [8, N] statistics), the gradient reads them and writes the
    gradient once."""
    import torch

    import blockwise_online_softmax_amd as ra

    N, V, t = 8192, 128256, 8
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda")
    g.manual_seed(88)
    z = (torch.randn((N, V), generator=g, device="cuda") * 3.0).to(torch.bfloat16)
    tg = torch.randint(0, V, (N,), generator=g, device="cuda", dtype=torch.int64)
    loss = torch.empty(N, dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ra_vocab_ce_workspace_bytes(N, t), dtype=torch.uint8, device="cuda")
    grad = torch.empty_like(z)
    ms = timed(lambda: ra.ra_vocab_ce(z, tg, t, loss, mean, lse, ws, stream=stream), args.steps,
               args.warmup, stream)
    nbytes = N * V * 2 + N * 8 + 3 * t * N * 4 * 2 + N * 8
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "ra_vocab_ce forward HBM GB/s (bf16 logits, 8 shards)", "rows": N, "vocab": V,
        "shards": t, "us_per_call": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
        "gb_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "steps": args.steps, "data": "synthetic"}), flush=True)
    ms = timed(lambda: ra.ra_vocab_ce_grad(z, tg, lse, 0, 1.0 / N, grad, stream=stream),
               args.steps, args.warmup, stream)
    nbytes = 2 * N * V * 2 + N * 12
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "ra_vocab_ce_grad HBM GB/s (bf16 logits and gradient)", "rows": N, "vocab": V,
        "us_per_call": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
        "gb_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "steps": args.steps, "data": "synthetic"}), flush=True)


def tiny_latency(args):
    """The pages' tiny case (4 devices x 3 tokens, d = 8, fp32, non-causal):
    microseconds per ra_ring call, HIP events on the launch stream."""
    import torch

    import blockwise_online_softmax_amd as ra
    import workloads

    q, k, v = (t.cuda() for t in workloads.workload_inputs("tiny"))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ms = timed(lambda: ra.ra_ring(q, k, v, out, lse, 4, "contiguous", False, -1, None,
                                  stream=stream), 1000, 50, stream)
    # the same call captured 100 times in one HIP graph: per-call time without
    # the host-side launch of each call
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        ra.ra_ring(q, k, v, out, lse, 4, "contiguous", False, -1, None)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(100):
            ra.ra_ring(q, k, v, out, lse, 4, "contiguous", False, -1, None)
    gms = timed(graph.replay, 10, 3, stream)
    print(json.dumps({"metric": "ra_ring latency, pages' tiny case (N=4 x 3 tokens, d=8, fp32)",
                      "us_per_call": round(ms * 1e3, 2), "calls": 1000,
                      "us_per_call_in_graph": round(gms * 1e3 / 100, 2),
                      "graph": "100 calls per graph, 10 replays"}), flush=True)


def xcd_ab(args):
    """The XCD split's effect on one workload, in one process: warm up with
    measuring on, freeze the measured speeds, then time `steps` launches under
    the even split and `steps` under the measured split, four times each, in
    the order even-split, split-even, ... so that a drift of the GPU's speed
    over the run cancels (HIP events around each launch)."""
    import torch

    import blockwise_online_softmax_amd as ra
    import workloads

    wkey, layout, device = WORKLOADS[args.workload]
    cfg = workloads.WORKLOADS[wkey]
    print(f"# generating inputs for {args.workload}", file=sys.stderr, flush=True)
    q, k, v = (t.cuda() for t in workloads.workload_inputs(wkey))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    nws = ra.ra_ring_workspace_bytes(q, k, cfg["N"], layout, device)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    stream = torch.cuda.current_stream()

    def step():
        ra.ra_ring(q, k, v, out, lse, cfg["N"], layout, cfg["causal"], device, ws, stream=stream)

    ra.ra_xcd_speeds(measure=True)  # measure from equal speeds
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < max(args.warmup, 16) or time.perf_counter() - t_w < 1.0:
        step()
        torch.cuda.synchronize()
        n_warm += 1
    speeds, nmeas = ra.ra_xcd_speeds()
    res = {"even": [], "split": []}
    try:
        for rep in range(4):
            pair = (("even", [1.0] * 8), ("split", speeds))
            for name, sp in (pair if rep % 2 == 0 else pair[::-1]):
                ra.ra_xcd_speeds(sp, set=True)
                res[name].append(timed(step, args.steps, 2, stream, stats=True)["mean"])
    finally:
        ra.ra_xcd_speeds(None, set=True)
    grid, M, keep, dbeg, dcnt = ra.ra_xcd_plan(q, k, cfg["N"], layout, cfg["causal"], device, speeds)
    even, split = float(np.mean(res["even"])), float(np.mean(res["split"]))
    print(json.dumps({
        "metric": "ring-attention launch ms, even split over the XCDs vs split by measured speed",
        "workload": args.workload, "speeds": [round(x, 4) for x in speeds], "measurements": nmeas,
        "warmup_calls": n_warm, "items_per_xcd": M, "items_moved": int(sum(dcnt)), "workgroups": grid,
        "even_ms": [round(x, 4) for x in res["even"]], "split_ms": [round(x, 4) for x in res["split"]],
        "gain": round(even / split - 1.0, 4),
    }), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   f"(got {args.gpus})"}))
        sys.exit(2)
    import torch

    import blockwise_online_softmax_amd as ra
    import workloads

    ra.load()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.tile_mix:
        tile_mix(args)
        return
    if args.step_sweep:
        step_sweep(args)
        return
    if args.layout_balance:
        layout_balance(args)
        return
    if args.tiny:
        tiny_latency(args)
        return
    if args.xcd_ab:
        xcd_ab(args)
        return
    if args.merge:
        merge_bench(args)
        return
    if args.vocab_ce:
        vocab_ce_bench(args)
        return
    wkey, layout, device = WORKLOADS[args.workload]
    cfg = workloads.WORKLOADS[wkey]
    S, N, D, Hq, Hkv = cfg["S"], cfg["N"], cfg["D"], cfg["Hq"], cfg["Hkv"]
    causal = cfg["causal"]
    print(f"# generating inputs for {args.workload}", file=sys.stderr, flush=True)
    q, k, v = workloads.workload_inputs(wkey)
    if device >= 0:
        pass  # share1m is drawn directly in device order (K, V) and local order (Q)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    nws = ra.ra_ring_workspace_bytes(qd, kd, N, layout, device)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    stream = torch.cuda.current_stream()

    def step():
        ra.ra_ring(qd, kd, vd, out, lse, N, layout, causal, device, ws, stream=stream)

    # warm-up: `warmup` calls, then more until 0.5 s have passed (the shader
    # clock ramps under load).  With --xcd measured, the warm-up launches
    # measure the XCD speeds (synchronised, so each launch's stamps land
    # before the next call), and the split is then frozen: the timed launches
    # enqueue the kernel and nothing else.
    if args.xcd == "measured":
        ra.ra_xcd_speeds(measure=True)
    else:
        ra.ra_xcd_speeds(None, set=True)
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < 0.5:
        step()
        torch.cuda.synchronize()
        n_warm += 1
    speeds, nmeas = ra.ra_xcd_speeds()
    if args.xcd == "measured":
        ra.ra_xcd_speeds(speeds, set=True)  # freeze
    for _ in range(2):  # first launches under the frozen split
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = wall * 1e3 / args.steps
    pairs = visible_pairs(S, N, layout, causal, device)
    flops = 4.0 * D * cfg["B"] * Hq * pairs
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    kern_ms = float(np.mean(ev_ms))
    kern_tflops = flops / (kern_ms * 1e-3) / 1e12
    q_tokens = qd.shape[2]
    props = torch.cuda.get_device_properties(0)

    grid, M, keep, dbeg, dcnt = ra.ra_xcd_plan(qd, kd, N, layout, causal, device, speeds)
    xcd = {"mode": args.xcd, "speeds": [round(x, 4) for x in speeds], "measurements": nmeas,
           "workgroups": grid, "items_per_xcd": M, "items_moved": int(sum(dcnt))}
    ra.ra_xcd_speeds(None, set=True)
    exec_flops = 4.0 * D * cfg["B"] * Hq * executed_pairs(S, N, layout, causal, device, D,
                                                          G=Hq // Hkv)
    ceiling = mfma_ceiling()
    ceiling["attention_kernel_frac_of_ceiling"] = round(kern_tflops / ceiling["tflops"], 4)
    cpu = None
    errs = None
    if not args.no_cpu_baseline:
        print("# timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        cpu, errs = cpu_baseline(q, k, v, cfg, layout, device, args.cpu_seconds,
                                 out.cpu(), lse.cpu())
    line = {
        "metric": "ring-attention TFLOP/s and % bf16 MFMA peak on 1 MI355X; tokens/s per ring",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": n_warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "batch": cfg["B"], "seq_len": S, "ring_devices": N, "q_heads": Hq, "kv_heads": Hkv,
            "head_dim": D, "causal": causal, "layout": layout, "device": device,
            "query_tokens": q_tokens, "seed": cfg["seed"], "parallelism": "1 GPU, N virtual",
        },
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(q_tokens / (ms_per_step * 1e-3), 1),
        "algorithmic_tflop": round(flops / 1e12, 4),
        "executed_tflop": round(exec_flops / 1e12, 4),
        "executed_over_algorithmic": round(exec_flops / flops, 4),
        "roofline": {
            "bound": "mfma", "achieved": round(kern_tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_traffic(args.workload),
            "kernel_ms": round(kern_ms, 4),
        },
        "launch_ms": ms_stats(ev_ms),
        "xcd_split": xcd,
        "mfma_ceiling": ceiling,
        "cpu_baseline": cpu,
        "sampled_max_err": None if errs is None else {"out": errs[0], "lse": errs[1]},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
