#!/usr/bin/env python3
"""Benchmark of the bounded tile-movement path on one MI355X.

A step is one pass over the bounded 2-D tile copy workload: bf16 matrix of
logical shape (8191, 4097) with row stride 4103, swept by (64, 32) tiles over
the ceil-div grids based at (0, 0) and (-16, -16); each sweep zero-fills a
dense tile buffer (tile_copy_bounded) and clip-stores it back into a second
matrix of the same layout (tile_store_clipped).  `value` is effective HBM GB/s
over algorithmic bytes (valid elements read, every tile slot written by the
copy; valid elements read and written by the store).

The same run also measures the other workloads of the path (row gather,
masked gather, masked scatter, ragged varlen load at group 1 and 4, bounded
GEMM) and reports them under "ops"; the CPU oracle is timed on the host on the
headline step ("cpu_baseline").  Inputs are synthetic and seeded, resident in
HBM before timing starts.

One GPU only: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, TFLOP/s
FP4_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default="all",
                    help="comma list of: copy,full,gather,masked,backward,zipf,ragged,gemm,scaled,calib (rocprof runs); 'all' for the "
                         "full report")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU time budget of the oracle baseline")
    ap.add_argument("--spinup-ms", type=float, default=400.0,
                    help="before each workload's warmup, run its step for this long (untimed) so the GPU's clocks "
                         "leave their idle state; 0 disables")
    return ap.parse_args()


def _dev(x, bf16=False):
    import torch

    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(x).to("cuda:0")


def source_hash(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_files, profile_name, label):
    """HBM bytes per launch of kernel `label` from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE runs, scaled by a plain copy of
    known size), if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    m = re.search(r"traffic_record:\s*(\{.*\})", open(path).read())
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_hash") != source_hash(*kernel_files):
        return None
    return rec.get("hbm_bytes_per_launch", {}).get(label)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def copy_workload(stg, inputs):
    import torch

    w = inputs.bounded_copy()
    M, N, ld = w["M"], w["N"], w["ld"]
    tm, tn = w["tile"]
    src = _dev(w["src"])[:, :N]
    dsts = [_dev(w["dst"])[:, :N] for _ in w["origins"]]
    bufs = []
    for (r0, c0) in w["origins"]:
        gr, gc = stg.stg_tile_grid(M, r0, tm), stg.stg_tile_grid(N, c0, tn)
        bufs.append(torch.empty((gr, gc, tm, tn), dtype=torch.bfloat16, device="cuda:0"))
    valid = M * N * 2
    kernels = []
    algo = {}
    for k, (r0, c0) in enumerate(w["origins"]):
        cn, sn = f"tile_copy_bounded@{r0},{c0}", f"tile_store_clipped@{r0},{c0}"
        kernels.append((cn, (lambda b=bufs[k], r0=r0, c0=c0: stg.tile_copy_bounded(src, tm, tn, r0, c0, out=b))))
        kernels.append((sn, (lambda b=bufs[k], d=dsts[k], r0=r0, c0=c0: stg.tile_store_clipped(b, r0, c0, d))))
        algo[cn] = valid + bufs[k].numel() * 2
        algo[sn] = 2 * valid
    return w, kernels, algo


SPINUP_MS = 0.0


def spin_up(fn):
    """Run `fn` repeatedly, untimed, for SPINUP_MS of wall time.  An idle
    MI355X starts a burst of work at reduced clocks and reaches its steady
    state only after tens of milliseconds under load; without this the timed
    steps of a short workload would measure the ramp, not the kernels."""
    import torch

    if SPINUP_MS <= 0:
        return
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SPINUP_MS:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def run_copy(stg, inputs, steps, warmup):
    """Time `steps` headline steps between two events on the launch stream,
    untraced.  Then repeat the same steps with the library's kernel tracing on
    (start/stop events inside each dispatch) for the per-kernel durations,
    which exclude the gaps between dependent launches; tracing itself widens
    those gaps, so the traced pass is never used for the step time."""
    import torch

    w, kernels, algo = copy_workload(stg, inputs)
    names = [n for n, _ in kernels]
    spin_up(lambda: [fn() for _, fn in kernels])
    for _ in range(warmup):
        for _, fn in kernels:
            fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        for _, fn in kernels:
            fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(end) / steps
    stg.stg_trace_read()
    stg.stg_trace_enable(True)
    for _ in range(steps):
        for _, fn in kernels:
            fn()
    torch.cuda.synchronize()
    stg.stg_trace_enable(False)
    trace = stg.stg_trace_read()
    if len(trace) != steps * len(kernels):
        raise RuntimeError(f"expected {steps * len(kernels)} traced launches, got {len(trace)}")
    per = {n: 0.0 for n in names}
    for i, (kname, ms) in enumerate(trace):
        label = names[i % len(names)]
        if not label.startswith(kname):
            raise RuntimeError(f"trace order mismatch: {kname} vs {label}")
        per[label] += ms / steps
    step_bytes = sum(algo.values())
    cold = cold_entry(stg, step_bytes, lambda: [fn() for _, fn in kernels], labels=names)
    return {"w": w, "per_kernel_ms": per, "algo": algo, "step_ms": step_ms, "wall_ms": wall * 1e3 / steps,
            "step_bytes": step_bytes, "cold": cold}


def time_fn(fn, iters, warmup):
    import torch

    spin_up(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


_FLUSH_W = None
_FLUSH_R = None


def flush_caches(i):
    """Evict L2 and the 256 MB Infinity Cache, leaving them clean: write a
    1 GiB buffer, then read a different 1 GiB buffer (a max-reduction into one
    value), so that the dirty lines of the write are written back during the
    read and the caches end up holding clean lines of the read buffer.  The
    timed call after it therefore pays no write-back of the flush's data."""
    import torch

    global _FLUSH_W, _FLUSH_R
    if _FLUSH_W is None:
        _FLUSH_W = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        _FLUSH_R = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
    _FLUSH_W.fill_(i & 0xFF)
    _FLUSH_R.max()


def cold_call_ms(stg, fn, calls=20, labels=None):
    """Per-call times with cold, clean caches (flush_caches before each call,
    outside the timed region); each call is bracketed by its own events on the
    launch stream and followed by a synchronize.  A second pass of the same
    calls with the library's dispatch tracing on gives each kernel's own
    duration with cold caches.  Returns ((median, min, max) in ms, {kernel:
    median ms})."""
    import torch

    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(calls):
        flush_caches(i)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    per = {}
    stg.stg_trace_read()
    for i in range(calls):
        flush_caches(i)
        torch.cuda.synchronize()
        stg.stg_trace_enable(True)
        fn()
        torch.cuda.synchronize()
        stg.stg_trace_enable(False)
        seen = {}
        trace = stg.stg_trace_read()
        if labels is not None and len(trace) != len(labels):
            raise RuntimeError(f"expected {len(labels)} traced launches, got {len(trace)}")
        for j, (kname, kms) in enumerate(trace):
            key = kname if labels is None else labels[j]
            seen[key] = seen.get(key, 0.0) + kms
        for kname, kms in seen.items():
            per.setdefault(kname, []).append(kms)
    kern = {k: round(sorted(v)[len(v) // 2], 5) for k, v in per.items()}
    return (times[len(times) // 2], times[0], times[-1]), kern


def cold_entry(stg, nbytes, fn, calls=20, flop=None, labels=None):
    (med, lo, hi), kern = cold_call_ms(stg, fn, calls, labels)
    e = {"median_ms": round(med, 5), "min_ms": round(lo, 5), "max_ms": round(hi, 5), "calls": calls,
         "kernel_median_ms": kern, "flush": "1 GiB written, then a different 1 GiB read, before each call"}
    if flop is None:
        e["GBps_at_median"] = round(gbs(nbytes, med), 1)
        e["kernel_GBps"] = round(gbs(nbytes, sum(kern.values())), 1) if kern else None
    else:
        e["TFLOPs_at_median"] = round(flop / (med * 1e-3) / 1e12, 1)
        e["kernel_TFLOPs"] = round(flop / (sum(kern.values()) * 1e-3) / 1e12, 1) if kern else None
    return e


def traced_kernel_ms(stg, fn, steps):
    """Per-kernel GPU durations (ms per call) of `fn`, from the library's
    dispatch tracing (start/stop events inside each dispatch)."""
    import torch

    torch.cuda.synchronize()
    stg.stg_trace_read()
    stg.stg_trace_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    stg.stg_trace_enable(False)
    kern = {}
    for kname, kms in stg.stg_trace_read():
        kern[kname] = kern.get(kname, 0.0) + kms / steps
    return {k: round(v, 5) for k, v in kern.items()}


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


ORACLE_OPS = True  # time the oracle beside each op (off with --no-cpu-baseline)
ORACLE_SECONDS = 1.5


def oracle_leg(fn, amount, unit, sample, seconds=None):
    """The CPU oracle as it stands, single-threaded and pinned to one host
    core, running `fn` (one bounded sample of an op's workload, `amount`
    algorithmic bytes or flop) repeatedly for about ORACLE_SECONDS.  A
    reported baseline, not a target."""
    if not ORACLE_OPS:
        return None
    allowed = sorted(os.sched_getaffinity(0))
    pinned = allowed[-1]
    os.sched_setaffinity(0, {pinned})
    try:
        n = 0
        t0 = time.perf_counter()
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= (seconds or ORACLE_SECONDS):
                break
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, set(allowed))
    rate = amount * n / dt
    value = rate / 1e12 if unit == "TFLOP/s" else rate / 1e9
    return {"value": round(value, 6 if unit == "TFLOP/s" else 3), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{sample}; {n} run(s) in {dt:.2f} s on host core {pinned} (pinned)"}


def op_entry(workload, nbytes, ms, kernel_ms=None):
    v = gbs(nbytes, ms)
    e = {"workload": workload, "value": round(v, 1), "unit": "GB/s", "ms": round(ms, 5),
         "algorithmic_bytes": int(nbytes), "frac_of_hbm_peak": round(v / HBM_PEAK_GBS, 4)}
    if kernel_ms:
        kt = sum(kernel_ms.values())
        e["kernel_ms"] = kernel_ms
        e["kernel_GBps"] = round(gbs(nbytes, kt), 1)
    return e


def run_full_tiles(stg, steps, warmup):
    """The unchecked full-tile path: bf16 (16384, 4096), row stride 4096, (64, 32)
    tiles from (0, 0) -- every tile is full, so the copy and the store take the
    instance without validity tests.  One call = copy + store; the working set
    (source, tiles, destination: 403 MB) exceeds the 256 MB Infinity Cache, as
    the headline step's does."""
    import torch

    M, N, tm, tn = 16384, 4096, 64, 32
    g = torch.Generator(device="cpu").manual_seed(1006)
    src = torch.randn((M, N), generator=g, dtype=torch.float32).to(torch.bfloat16).to("cuda:0")
    dst = torch.empty_like(src)
    tiles = torch.empty((M // tm, N // tn, tm, tn), dtype=torch.bfloat16, device="cuda:0")

    def fn():
        stg.tile_copy_windows(src, tm, tn, tm, tn, 0, 0, check_bounds=False, out=tiles)
        stg.tile_store_windows(tiles, tm, tn, 0, 0, dst, check_bounds=False)

    ms = time_fn(fn, steps, warmup)
    kms = traced_kernel_ms(stg, fn, steps)
    nbytes = 4 * M * N * 2  # copy: read + write every element; store: the same
    e = op_entry("full-tile copy + store, unchecked: bf16 (16384,4096) ld 4096, (64,32) tiles from (0,0)", nbytes,
                 ms, kms)
    e["cold_cache"] = cold_entry(stg, nbytes, fn)
    if ORACLE_OPS:
        import oracle

        ms_rows = 1024
        src_h = src[:ms_rows].view(torch.int16).cpu().numpy().view(np.uint16)
        dst_h = np.empty_like(src_h)

        def orc_fn():
            t = oracle.tile_copy_windows(src_h, tm, tn, tm, tn, 0, 0)
            oracle.tile_store_windows(t, tm, tn, 0, 0, dst_h)

        e["cpu_baseline"] = oracle_leg(orc_fn, 4 * ms_rows * N * 2, "GB/s",
                                       f"copy + store of the first {ms_rows} rows (same tiles)")
    return e


def run_gather(stg, inputs, steps, warmup):
    w = inputs.row_gather()
    a, idx = _dev(w["a"]), _dev(w["indices"])
    import torch

    out = torch.empty((idx.numel(), w["a"].shape[1]), dtype=torch.float32, device="cuda:0")
    fn = lambda: stg.tile_gather(a, idx, w["tile_shape"], w["offset"], w["axis"], out=out)
    # a call is a few microseconds: time at least 200, so that one hiccup of
    # the host or the driver does not dominate the mean
    ms = time_fn(fn, max(steps, 200), warmup)
    kms = traced_kernel_ms(stg, fn, steps)
    n_valid = int(((w["indices"] >= 0) & (w["indices"] < w["a"].shape[0])).sum())
    row_b = w["a"].shape[1] * 4
    nbytes = idx.numel() * 4 + n_valid * row_b + idx.numel() * row_b
    e = op_entry("row gather fp32 (1024,256), 4096 int32 indices in [-64,1087], (64,256) tiles", nbytes, ms, kms)
    e["cold_cache"] = cold_entry(stg, nbytes, fn)
    e["note"] = "about 8 MB per call: bound by launch latency and host call overhead, not by HBM"
    e["graph_replay"] = graph_replay(fn, nbytes, steps)
    # the same call prepared once (argument marshalling done at preparation):
    # eager calls back to back
    call = stg.prepare(stg.tile_gather, a, idx, w["tile_shape"], w["offset"], w["axis"], out=out)
    pms = time_fn(call, max(steps, 200), warmup)
    e["prepared_call"] = {"us_per_call": round(pms * 1e3, 3), "GBps": round(gbs(nbytes, pms), 1),
                          "note": "stg.prepare(stg.tile_gather, ...): descriptors built once, one C call per step"}
    e["empty_dispatch_note"] = ("kernel_ms comes from start/stop events inside the dispatch; an empty kernel timed "
                                "the same way reads about 3.9 us on this GPU")
    if ORACLE_OPS:
        import oracle

        e["cpu_baseline"] = oracle_leg(
            lambda: oracle.tile_gather(w["a"], w["indices"], w["tile_shape"], w["offset"], w["axis"]), nbytes,
            "GB/s", "the whole workload")
    return e


def graph_replay(fn, nbytes, steps, calls=64):
    """Per-call time with `calls` calls captured in one HIP graph and the
    graph replayed `steps` times: the launch path without the host call."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    per_call = ev0.elapsed_time(ev1) / (steps * calls)
    return {"calls_per_graph": calls, "replays": steps, "us_per_call": round(per_call * 1e3, 3),
            "GBps": round(gbs(nbytes, per_call), 1)}


def run_masked(stg, inputs, steps, warmup):
    import torch

    w = inputs.masked()
    table, idx, gm = _dev(w["table"]), _dev(w["indices"]), _dev(w["gmask"])
    rows, cols = w["table"].shape
    out = torch.empty((idx.numel(), cols), dtype=torch.float32, device="cuda:0")
    fn = lambda: stg.tile_gather_masked(table, idx, gm, (64, cols), None, 0, w["padding_value"], out=out)
    ms_g = time_fn(fn, steps, warmup)
    kms_g = traced_kernel_ms(stg, fn, steps)
    n_true = int(w["gmask"].sum())
    row_b = cols * 4
    g_bytes = idx.numel() * 5 + n_true * row_b + idx.numel() * row_b
    cold_g = cold_entry(stg, g_bytes, fn)
    del out
    vals, perm, sm = _dev(w["vals"]), _dev(w["perm"]), _dev(w["smask"])
    dst = table.clone()
    fn = lambda: stg.tile_scatter_masked(dst, perm, sm, (64, cols), vals, None, 0)
    ms_s = time_fn(fn, steps, warmup)  # rewrites the same rows each call: same traffic
    kms_s = traced_kernel_ms(stg, fn, steps)
    s_true = int(w["smask"].sum())
    s_bytes = perm.numel() * 5 + 2 * s_true * row_b
    eg = op_entry("masked gather fp32 table (1048576,128), 4194304 indices, Bernoulli(0.9) mask, pad -1.0",
                  g_bytes, ms_g, kms_g)
    eg["cold_cache"] = cold_g
    es = op_entry("masked scatter fp32 (1048576,128) rows to a permutation, Bernoulli(0.5) mask", s_bytes, ms_s,
                  kms_s)
    es["cold_cache"] = cold_entry(stg, s_bytes, fn)
    if ORACLE_OPS:
        import oracle

        n = 262144
        si, sg = w["indices"][:n], w["gmask"][:n]
        nb = n * 5 + int(sg.sum()) * row_b + n * row_b
        eg["cpu_baseline"] = oracle_leg(
            lambda: oracle.tile_gather_masked(w["table"], si, sg, (64, cols), None, 0, w["padding_value"], "f32"), nb,
            "GB/s", f"the first {n} of the {idx.numel()} indices")
        dst_h = w["table"].copy()
        sp, ss, sv = w["perm"][:n], w["smask"][:n], w["vals"][:n]
        nb = n * 5 + 2 * int(ss.sum()) * row_b
        es["cpu_baseline"] = oracle_leg(
            lambda: oracle.tile_scatter_masked(dst_h, sp, ss, (64, cols), sv, None, 0), nb, "GB/s",
            f"the first {n} of the {perm.numel()} rows")
    return eg, es


def run_gather_backward(stg, inputs, steps, warmup):
    """Backward of the indexed gather at embedding scale: a.grad fp32
    (1048576, 128), the masked workload's 4,194,304 uniform indices (about
    four terms per row), an N(0,1) output gradient (4194304, 128), (64, 128)
    tiles.  Every call accumulates into the same a.grad."""
    import torch

    w = inputs.masked()
    idx = _dev(w["indices"])
    rows, cols = w["table"].shape
    g = torch.Generator(device="cuda:0").manual_seed(1007)
    grad_out = torch.randn((idx.numel(), cols), generator=g, dtype=torch.float32, device="cuda:0")
    a_grad = torch.zeros((rows, cols), dtype=torch.float32, device="cuda:0")
    touched = int(np.unique(w["indices"]).size)
    nbytes = idx.numel() * 4 + idx.numel() * cols * 4 + 2 * touched * cols * 4
    res = []
    nws = stg.tile_gather_backward_workspace(a_grad, idx.numel(), (64, cols), 0)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda:0")
    for label, wsp in (("grouped by destination row, no float atomics", ws), ("hardware fp32 atomic adds", None)):
        fn = lambda: stg.tile_gather_backward(a_grad, idx, (64, cols), grad_out, workspace=wsp)
        ms = time_fn(fn, steps, warmup)
        kms = traced_kernel_ms(stg, fn, steps)
        e = op_entry(f"gather backward ({label}): a.grad fp32 (1048576,128), 4194304 uniform indices, (64,128) "
                     f"tiles", nbytes, ms, kms)
        e["note"] = ("algorithmic bytes: indices, the output gradient read once, each touched a.grad row read "
                     "and written once")
        if wsp is not None:
            e["workspace_bytes"] = int(nws)
        e["cold_cache"] = cold_entry(stg, nbytes, fn)
        res.append(e)
    if ORACLE_OPS:
        res[0]["cpu_baseline"] = _backward_oracle(w["indices"], rows, cols)
        res[1]["cpu_baseline"] = dict(res[0]["cpu_baseline"], sample=res[0]["cpu_baseline"]["sample"] +
                                      " (the oracle has one execution; the same figure serves both legs)")
    return res


def _backward_oracle(idx_h, rows, cols, n=262144):
    """The oracle backward on the first n indices of an index list (one leg
    serves both executions: the oracle has one)."""
    import oracle

    si = idx_h[:n]
    g_h = np.random.default_rng(1007).standard_normal((n, cols), dtype=np.float32)
    a0 = np.zeros((rows, cols), dtype=np.float32)
    nb = n * 4 + n * cols * 4 + 2 * int(np.unique(si).size) * cols * 4
    return oracle_leg(lambda: oracle.tile_gather_backward(a0, si, (64, cols), g_h, None, 0), nb, "GB/s",
                      f"the first {n} of the {idx_h.size} indices (fp64 accumulation into a copy of a.grad)")


def run_gather_backward_zipf(stg, inputs, steps, warmup):
    """The grouped backward of the workload above on skewed indices: Zipf,
    a = 1.1 truncated to the table (the hottest row takes about 12% of the
    4,194,304 terms)."""
    import torch

    w = inputs.masked()
    rows, cols = w["table"].shape
    zidx_h = inputs.zipf_indices(rows=rows, n=w["indices"].size)
    zidx = _dev(zidx_h)
    g = torch.Generator(device="cuda:0").manual_seed(1007)
    grad_out = torch.randn((zidx.numel(), cols), generator=g, dtype=torch.float32, device="cuda:0")
    a_grad = torch.zeros((rows, cols), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(stg.tile_gather_backward_workspace(a_grad, zidx.numel(), (64, cols), 0), dtype=torch.uint8,
                     device="cuda:0")
    touched = int(np.unique(zidx_h).size)
    nbytes = zidx.numel() * 4 + zidx.numel() * cols * 4 + 2 * touched * cols * 4
    fn = lambda: stg.tile_gather_backward(a_grad, zidx, (64, cols), grad_out, workspace=ws)
    ms = time_fn(fn, steps, warmup)
    kms = traced_kernel_ms(stg, fn, steps)
    e = op_entry("gather backward (grouped by destination row), Zipf(1.1) indices: a.grad fp32 (1048576,128), "
                 "4194304 indices, (64,128) tiles", nbytes, ms, kms)
    e["note"] = ("algorithmic bytes as for the uniform indices; rows past 64 terms are split into pieces added with "
                 "float atomics")
    e["max_terms_per_row"] = int(np.bincount(zidx_h).max())
    e["cold_cache"] = cold_entry(stg, nbytes, fn)
    if ORACLE_OPS:
        e["cpu_baseline"] = _backward_oracle(zidx_h, rows, cols)
    return e


def run_ragged(stg, inputs, steps, warmup):
    import torch

    w = inputs.ragged()
    X = _dev(w["X"])
    res = []
    for group in (1, 4):
        md = w["heads"] // group
        ri, dyn, mi = stg.ragged_tile_schedule(w["seq_lens"], 128 // group, md)
        tri = [torch.from_numpy(x.astype(np.int32)).to("cuda:0") for x in (ri, dyn, mi)]
        out = torch.empty((len(ri), 128, 128), dtype=torch.bfloat16, device="cuda:0")
        fn = lambda: stg.ragged_tile_load(X, md, group, 128, 128, *tri, out=out)
        ms = time_fn(fn, steps, warmup)
        kms = traced_kernel_ms(stg, fn, steps)
        nbytes = w["X"].nbytes + out.numel() * 2 + len(ri) * 12
        e = op_entry(f"ragged varlen load bf16 ({w['X'].shape[0]},8,128), 64 seqs, BM=128, group={group}",
                     nbytes, ms, kms)
        e["cold_cache"] = cold_entry(stg, nbytes, fn)
        nt = 1024
        if ORACLE_OPS:
            import oracle

            sri, sdy, smi = ri[:nt], dyn[:nt], mi[:nt]
            nb = int(sdy.sum()) * group * 128 * 2 + nt * 128 * 128 * 2 + nt * 12
            e["cpu_baseline"] = oracle_leg(
                lambda: oracle.ragged_tile_load(w["X"], md, group, 128, 128, 0, sri, sdy, smi), nb, "GB/s",
                f"the first {nt} of the {len(ri)} tiles")
        res.append(e)
        # store direction: the loaded tiles back into a copy of X (every call
        # rewrites the same elements); the schedule covers every row and head
        # once, so the valid elements are all of X, read from the tiles once
        # and written once
        dst = X.clone()
        fn = lambda: stg.ragged_tile_store(out, dst, md, group, *tri)
        ms = time_fn(fn, steps, warmup)
        kms = traced_kernel_ms(stg, fn, steps)
        nbytes = 2 * w["X"].nbytes + len(ri) * 12
        e = op_entry(f"ragged varlen store bf16 ({w['X'].shape[0]},8,128), 64 seqs, BM=128, group={group}",
                     nbytes, ms, kms)
        e["cold_cache"] = cold_entry(stg, nbytes, fn)
        if ORACLE_OPS:
            tiles_h = out[:nt].view(torch.int16).cpu().numpy().view(np.uint16)
            nb = 2 * int(sdy.sum()) * group * 128 * 2 + nt * 12
            e["cpu_baseline"] = oracle_leg(
                lambda: oracle.ragged_tile_store(tiles_h, w["X"], md, group, 0, sri, sdy, smi), nb, "GB/s",
                f"the first {nt} of the {len(ri)} tiles (the oracle stores into a fresh copy of X per run, "
                f"not timed apart)")
        res.append(e)
        del out, dst
    return res


def run_gemm(stg, inputs, steps, warmup):
    import torch

    M, N, K = 8191, 8193, 4097
    g = inputs.gemm(M, N, K)
    A, B = _dev(g["A"]), _dev(g["B"])
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    fn = lambda: stg.gemm_bounded(A, B, out=C)
    try:
        fn()
    except Exception as e:  # reported, not hidden
        return {"workload": "bounded GEMM bf16 (8191,8193,4097)", "error": str(e)}
    ms = time_fn(fn, steps, warmup)
    kern = traced_kernel_ms(stg, fn, steps)
    flop = 2.0 * M * N * K
    tf = flop / (ms * 1e-3) / 1e12
    e = {"workload": "bounded GEMM bf16 A(8191,4097) B(4097,8193), fp32 accumulate, bf16 clipped output",
         "value": round(tf, 1), "unit": "TFLOP/s", "ms": round(ms, 4), "flop": flop,
         "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
         "kernel_ms": kern,
         "cold_cache": cold_entry(stg, 0, fn, flop=flop)}
    if ORACLE_OPS:
        import oracle

        pr = 16
        Ap = np.ascontiguousarray(g["A"][:pr])
        e["cpu_baseline"] = oracle_leg(lambda: oracle.gemm_f64(Ap, g["B"]), 2.0 * pr * N * K, "TFLOP/s",
                                       f"one {pr}-row panel of the {M}-row output (fp64 sums), extrapolated to "
                                       f"the whole GEMM as a rate")
    return e


def run_gemm_aligned(stg, inputs, steps, warmup):
    """The same GEMM at 8192 x 8192 x 4096, where every operand row starts
    16-byte aligned (the 4-wave main kernel; no K edge, no remainder columns),
    beside hipBLASLt (torch.matmul) on the same operands and output."""
    import torch

    M, N, K = 8192, 8192, 4096
    g = inputs.gemm(M, N, K)
    A, B = _dev(g["A"]), _dev(g["B"])
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    fn = lambda: stg.gemm_bounded(A, B, out=C)
    ms = time_fn(fn, steps, warmup)
    kern = traced_kernel_ms(stg, fn, steps)
    lib = lambda: torch.matmul(A.view(torch.bfloat16), B.view(torch.bfloat16), out=C)
    lib_ms = time_fn(lib, steps, warmup)
    flop = 2.0 * M * N * K
    tf = flop / (ms * 1e-3) / 1e12
    return {"workload": "bounded GEMM bf16 A(8192,4096) B(4096,8192), aligned rows, fp32 accumulate, bf16 output",
            "value": round(tf, 1), "unit": "TFLOP/s", "ms": round(ms, 4), "flop": flop,
            "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4), "kernel_ms": kern,
            "hipblaslt_same_call": {"value": round(flop / (lib_ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                                    "ms": round(lib_ms, 4), "note": "torch.matmul on the same operands, context only"}}


def run_gemm_scaled(stg, inputs, steps, warmup):
    """Block-scaled GEMM, fp8 e4m3 and fp4 e2m1 operands with e8m0 scales per
    32 K values, fp32 output, on the bounded GEMM's odd M and N."""
    import torch

    M, N, K = 8191, 8193, 4096
    out = {}
    for fmt, peak in (("e4m3", FP8_PEAK_TFLOPS), ("e2m1", FP4_PEAK_TFLOPS)):
        g = inputs.scaled_gemm(M, N, K, fmt)
        A, Bt, sa, sb = _dev(g["A"]), _dev(g["Bt"]), _dev(g["sa"]), _dev(g["sb"])
        C = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        fn = lambda: stg.gemm_scaled(A, fmt, sa, Bt, fmt, sb, K, 32, out=C)
        name = f"gemm_scaled_{'fp8' if fmt == 'e4m3' else 'fp4'}"
        try:
            fn()
        except Exception as e:  # reported, not hidden
            out[name] = {"workload": f"block-scaled GEMM {fmt} (8191,8193,4096)", "error": str(e)}
            continue
        ms = time_fn(fn, steps, warmup)
        kern = traced_kernel_ms(stg, fn, steps)
        flop = 2.0 * M * N * K
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = {"workload": f"block-scaled GEMM {fmt} x {fmt}, e8m0 scales per 32 K values, A(8191,4096) "
                                 f"Bt(8193,4096), fp32 clipped output",
                     "value": round(tf, 1), "unit": "TFLOP/s", "ms": round(ms, 4), "flop": flop,
                     "frac_of_peak": round(tf / peak, 4), "peak_tflops": peak, "kernel_ms": kern,
                     "cold_cache": cold_entry(stg, 0, fn, flop=flop)}
        if ORACLE_OPS:
            import oracle

            pr = 2
            Ap, sap = np.ascontiguousarray(g["A"][:pr]), np.ascontiguousarray(g["sa"][:pr])
            out[name]["cpu_baseline"] = oracle_leg(
                lambda: oracle.gemm_scaled_f64(Ap, fmt, sap, g["Bt"], fmt, g["sb"], K, 32), 2.0 * pr * N * K,
                "TFLOP/s", f"one {pr}-row panel of the {M}-row output (fp64 sums of decoded values), extrapolated "
                           f"to the whole GEMM as a rate")
        del A, Bt, sa, sb, C
    # the general path: e4m3 scales per 16 values (no scaled-MFMA layout);
    # with a workspace, each operand decoded to bf16 once and multiplied by
    # the bf16 GEMM, and beside it the fused kernel (values scaled while
    # staged, bf16 MFMA, no workspace); fp8 e4m3 values, and fp4 e2m1 values
    # (two per byte) -- e2m1 with e4m3 scales per 16 is the layout of the
    # 4-bit formats that scale every 16 values
    for fmt, key, what in (("e4m3", "gemm_scaled_general_fp8_e4m3scales", "e4m3 x e4m3"),
                           ("e2m1", "gemm_scaled_general_fp4_e4m3scales", "e2m1 x e2m1 (two per byte)")):
        g = inputs.scaled_gemm(M, N, K, fmt, block=16)
        rng = np.random.default_rng(1016)
        sa_h = rng.integers(0x28, 0x48, g["sa"].shape).astype(np.uint8)  # e4m3 scales 2^-2 .. 2^2 x (1 + m/8)
        sb_h = rng.integers(0x28, 0x48, g["sb"].shape).astype(np.uint8)
        A, Bt, sa, sb = _dev(g["A"]), _dev(g["Bt"]), _dev(sa_h), _dev(sb_h)
        C = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        ws = torch.empty(stg.gemm_scaled_workspace(fmt, fmt, "e4m3", 16, M, N, K), dtype=torch.uint8,
                         device="cuda:0")
        fn = lambda: stg.gemm_scaled(A, fmt, sa, Bt, fmt, sb, K, 16, scale_fmt="e4m3", out=C, workspace=ws)
        fused = lambda: stg.gemm_scaled(A, fmt, sa, Bt, fmt, sb, K, 16, scale_fmt="e4m3", out=C, workspace=None)
        fn()
        fused()
        ms = time_fn(fn, steps, warmup)
        kern = traced_kernel_ms(stg, fn, steps)
        ms_f = time_fn(fused, steps, warmup)
        flop = 2.0 * M * N * K
        tf = flop / (ms * 1e-3) / 1e12
        out[key] = {
            "workload": f"block-scaled GEMM {what} with e4m3 scales per 16 K values (general path: each operand "
                        "decoded to bf16 once into a workspace, then the bf16 GEMM), A(8191,4096) Bt(8193,4096), fp32 "
                        "clipped output",
            "value": round(tf, 1), "unit": "TFLOP/s", "ms": round(ms, 4), "flop": flop,
            "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4), "kernel_ms": kern,
            "workspace_bytes": ws.numel(),
            "fused_no_workspace": {"value": round(flop / (ms_f * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                                   "ms": round(ms_f, 4),
                                   "note": "values scaled while staged inside the GEMM kernel (bf16 MFMA)"},
            "cold_cache": cold_entry(stg, 0, fn, flop=flop)}
        if ORACLE_OPS:
            import oracle

            pr = 2
            Ap, sap = np.ascontiguousarray(g["A"][:pr]), np.ascontiguousarray(sa_h[:pr])
            out[key]["cpu_baseline"] = oracle_leg(
                lambda: oracle.gemm_scaled_f64(Ap, fmt, sap, g["Bt"], fmt, sb_h, K, 16, s_fmt="e4m3"),
                2.0 * pr * N * K, "TFLOP/s", f"one {pr}-row panel of the {M}-row output, extrapolated to the whole "
                                             f"GEMM as a rate")
        del A, Bt, sa, sb, C, ws
    return out


def run_calibration(steps):
    """A plain device-to-device copy of a known size (512 MiB read, 512 MiB
    written), for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read": n, "bytes_written": n, "launches": steps}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inputs, budget_s):
    """The oracle, single-threaded and pinned to one host core, on the
    headline step."""
    import oracle

    allowed = sorted(os.sched_getaffinity(0))
    pinned = allowed[-1]
    os.sched_setaffinity(0, {pinned})
    try:
        res = _cpu_baseline_run(oracle, inputs, budget_s)
    finally:
        os.sched_setaffinity(0, set(allowed))
    res["pinned_core"] = pinned
    res["host_cores_available"] = len(allowed)
    res["cpu_model"] = cpu_model()
    return res


def _cpu_baseline_run(oracle, inputs, budget_s):
    w = inputs.bounded_copy()
    M, N = w["M"], w["N"]
    tm, tn = w["tile"]
    src = w["src"][:, :N]
    dst = w["dst"].copy()
    step_bytes = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        for (r0, c0) in w["origins"]:
            tiles = oracle.tile_copy_bounded(src, tm, tn, r0, c0)
            oracle.tile_store_clipped(tiles, r0, c0, dst[:, :N])
            if steps == 0:
                step_bytes += M * N * 2 + tiles.nbytes + 2 * M * N * 2
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(step_bytes * steps / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full headline steps (copy + clipped store at both grid bases), "
                      f"{dt:.1f} s on one host core (pinned)"}


def main():
    global SPINUP_MS, ORACLE_OPS
    args = parse()
    SPINUP_MS = args.spinup_ms
    ORACLE_OPS = not args.no_cpu_baseline
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); nothing run.", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import scatter_tile_gather_amd as stg
    from scatter_tile_gather_amd import inputs

    stg.load_library()
    only = set(args.only.split(",")) if args.only != "all" else {"copy", "full", "gather", "masked", "backward", "zipf",
                                                                             "ragged", "gemm", "scaled"}
    ops = {}
    head = None
    if "calib" in only:
        ops["calibration_copy"] = run_calibration(args.steps)
    if "copy" in only:
        head = run_copy(stg, inputs, args.steps, args.warmup)
        print(f"[bench] copy step {head['step_ms']:.4f} ms", file=sys.stderr, flush=True)
    if "full" in only:
        ops["full_tile_unchecked"] = run_full_tiles(stg, args.steps, args.warmup)
        print("[bench] full-tile unchecked done", file=sys.stderr, flush=True)
    if "gather" in only:
        ops["row_gather"] = run_gather(stg, inputs, args.steps, args.warmup)
        print("[bench] row gather done", file=sys.stderr, flush=True)
    if "masked" in only:
        ops["masked_gather"], ops["masked_scatter"] = run_masked(stg, inputs, args.steps, args.warmup)
        print("[bench] masked gather/scatter done", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if "backward" in only:
        ops["gather_backward_grouped"], ops["gather_backward_atomic"] = run_gather_backward(stg, inputs, args.steps,
                                                                                            args.warmup)
        print("[bench] gather backward done", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if "zipf" in only:
        ops["gather_backward_grouped_zipf"] = run_gather_backward_zipf(stg, inputs, args.steps, args.warmup)
        print("[bench] gather backward, Zipf indices, done", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if "ragged" in only:
        (ops["ragged_group1"], ops["ragged_store_group1"], ops["ragged_group4"],
         ops["ragged_store_group4"]) = run_ragged(stg, inputs, args.steps, args.warmup)
        print("[bench] ragged done", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if "gemm" in only:
        ops["gemm_bounded"] = run_gemm(stg, inputs, max(args.steps // 2, 1), args.warmup)
        ops["gemm_bounded_aligned"] = run_gemm_aligned(stg, inputs, max(args.steps // 2, 1), args.warmup)
        print("[bench] gemm done", file=sys.stderr, flush=True)
    if "scaled" in only:
        ops.update(run_gemm_scaled(stg, inputs, max(args.steps // 2, 1), args.warmup))
        print("[bench] scaled gemm done", file=sys.stderr, flush=True)
    if head is None:
        print(json.dumps({"ops": ops}))
        return
    per = head["per_kernel_ms"]
    # the roofline kernel: the one of the step's four with the lowest achieved
    # rate (algorithmic bytes / average duration), i.e. the furthest from peak
    dom = min(per, key=lambda n: gbs(head["algo"][n], per[n]))
    achieved = gbs(head["algo"][dom], per[dom])
    cold_k = head["cold"]["kernel_median_ms"]
    traffic = traffic_from_profile(("scatter_tile_gather_amd/csrc/copy.hip", "scatter_tile_gather_amd/csrc/stg_internal.h"),
                                   "tile_copy_bounded.bounded_copy_workload.md", dom)
    value = gbs(head["step_bytes"], head["step_ms"])
    line = {
        "metric": "effective HBM GB/s (gather/copy/scatter, % of peak); bounded GEMM TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "bounded 2-D tile copy + clipped store: bf16 (8191,4097) row stride 4103, (64,32) tiles, "
                        "ceil-div grids based at (0,0) and (-16,-16)",
            "tiles_per_step": 16512 + 16641,
            "algorithmic_bytes_per_step": int(head["step_bytes"]),
            "step_host_wall_ms": round(head["wall_ms"], 5),
            "spinup_ms_before_warmup": args.spinup_ms,
            "per_kernel_ms": {k: round(v, 5) for k, v in per.items()},
            "dispatch_gaps_ms_per_step": round(head["step_ms"] - sum(per.values()), 5),
            "cold_cache_step": head["cold"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(head["algo"][dom]),
            "kernel_rule": "lowest achieved GB/s of the step's four kernels (warm, back-to-back steps)",
            "kernel_ms": round(per[dom], 5),
            "cold": {"kernel_ms": cold_k.get(dom), "achieved": round(gbs(head["algo"][dom], cold_k[dom]), 1),
                     "frac": round(gbs(head["algo"][dom], cold_k[dom]) / HBM_PEAK_GBS, 4),
                     "note": "the same kernel with caches flushed clean before each call (median of 20)"},
            "per_kernel_frac": {k: round(gbs(head["algo"][k], v) / HBM_PEAK_GBS, 4) for k, v in per.items()},
            "per_kernel_frac_cold": {k: round(gbs(head["algo"][k], v) / HBM_PEAK_GBS, 4) for k, v in cold_k.items()},
        },
        "ops": ops,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inputs, args.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
