#!/usr/bin/env python3
"""Benchmark of the MI355X Mamba2 selective-state scan (one layer's scan).

Headline: decode, 16 sequences x 1 token at H=64, P=64, N=128, G=8, fp32,
resuming state.  A step is one ssm_scan_decode call.  Consecutive steps use
16 disjoint slot sets of a 256-slot state (537 MB), so each step's 33.5 MB of
state comes from HBM, not from the 256 MB Infinity Cache.  After --warmup
untimed steps, exactly --steps launches are timed between HIP events; a spin
kernel enqueued ahead of the start event keeps the GPU busy while the host
enqueues them, so they run back to back and the timed region holds the
steps' kernels and the gaps between them only.  The same is done for a
hand-written read-modify-write stream over the same slot sets (the
achievable ceiling for a kernel that reads and writes each state value once).

Also measured and reported beside it: the 1 x 4096-token prefill at the same
geometry, both on the matrix cores (the automatic time split) and on the
VALU (the one-pass register kernel), the secondary scan workloads, the ops
beside the scan (conv1d + SiLU, gated RMSNorm), the gated delta rule, and the
fp32 CPU oracle on all five workloads at one thread and at every thread the
process may use.

Prints one JSON line.  Times come from HIP events on the stream the kernels run
on; the roofline objects use algorithmic bytes (decode, HBM-bound) and
algorithmic flops (prefill).  Figures from counter and kernel-trace runs
(HBM traffic, VALU and matrix-core busy, LDS bank conflicts, kernel-trace
medians) are read from committed summaries under profiles/ and only when they
were taken on the current kernel sources (a hash of them); else null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_VALU_PEAK_TFLOPS = 157.3  # 256 CU x 2.4 GHz x 256 flop/clk (packed FMA)
FP32_VALU_UNPACKED_TFLOPS = 78.6
FP32_MFMA_PEAK_TFLOPS = 157.3  # dense fp32 matrix (v_mfma_f32_*)
H, P, N, G = 64, 64, 128, 8
DECODE_SEQS, SLOT_SETS = 16, 16
PREFILL_T = 4096


def decode_bytes(n_seqs=DECODE_SEQS):
    """Algorithmic bytes of one decode launch: resumed state read + written,
    x, y, B, C, dt, A, slot, fresh -- each moved once."""
    state = n_seqs * H * P * N * 4
    return 2 * state + 2 * n_seqs * H * P * 4 + 2 * n_seqs * G * N * 4 + n_seqs * H * 4 \
        + H * 4 + n_seqs * 4 + n_seqs


def prefill_bytes(T=PREFILL_T):
    """x and y, B and C, dt, A, cu_seqlens/slot/fresh, final state write."""
    return 2 * T * H * P * 4 + 2 * T * G * N * 4 + T * H * 4 + H * 4 + 8 + 4 + 1 + H * P * N * 4


def prefill_flops(T=PREFILL_T):
    """5 flops per (token, head, row, state element): 2 multiplies and an add
    for the update, a multiply and an add for y."""
    return 5 * T * H * P * N


def kernel_source_hash():
    """Hash of what determines the kernels' machine code: the HIP sources and
    the C header with comments and whitespace removed, and the hipcc flags.
    Counter results are tied to it, so they stop counting once the code
    changes, but not when only a comment does."""
    import re
    h = hashlib.sha256()
    for rel in ("mamba2_selective_scan_amd/csrc/scan_kernel.hpp",
                "mamba2_selective_scan_amd/csrc/correct_mfma.hpp",
                "mamba2_selective_scan_amd/csrc/ssd_kernel.hpp",
                "mamba2_selective_scan_amd/csrc/decode_kernel.hpp",
                "mamba2_selective_scan_amd/csrc/buffer_io.hpp",
                "mamba2_selective_scan_amd/csrc/status.hpp",
                "mamba2_selective_scan_amd/csrc/ssm_scan.hip", "include/ssm_scan.h"):
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    with open(os.path.join(ROOT, "mamba2_selective_scan_amd", "build.py")) as f:
        flags = re.search(r"FLAGS = \[(.*?)\]", f.read(), re.S).group(1)
    h.update(" ".join(flags.split()).encode())
    return h.hexdigest()[:16]


def load_profile(name):
    """A committed summary under profiles/ (``<name>.json``) if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_hash") == kernel_source_hash() else None


def load_traffic(name):
    """Measured HBM bytes per launch from a committed counter run, if it was
    taken on the current kernel source; else None."""
    t = load_profile(f"{name}_traffic")
    return None if t is None else t.get("bytes_per_launch")


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


CPU_CONFIGS = (("decode16", "decode 16 x 1, resuming, H64 P64 N128 G8"),
               ("tiny", "tiny scan T64 H4 P16 N16 G1"),
               ("mixed", "mixed edge batch, 8 seqs / 523 tokens, H16 P96 N100 G4"),
               ("decode256", "decode 256 x 1, resuming, H64 P64 N128 G8"),
               ("prefill4096", "prefill 1 x 4096, fresh, H64 P64 N128 G8"))


def cpu_baseline(seconds):
    """The fp32 oracle (plain sequential C, OpenMP over (sequence, head)) on
    each of the five workloads, at one thread and at every thread the process
    may use; each timing repeats the whole workload until ``seconds`` have
    passed (at least once) and keeps the fastest run.  The fp64 oracle on all
    threads is informational.  Rank 0, one GPU only."""
    import oracle
    import ssm_inputs
    orc = oracle.default()
    threads = oracle.default_threads()

    def best(case, th, precision="f32"):
        runs, t_all = [], time.perf_counter()
        while True:
            t0 = time.perf_counter()
            orc.scan_case(case, precision=precision, threads=th)
            runs.append(time.perf_counter() - t0)
            if time.perf_counter() - t_all >= seconds:
                return min(runs), len(runs)
    per, total_s = {}, time.perf_counter()
    for name, desc in CPU_CONFIGS:
        case = ssm_inputs.workload(name)
        orc.scan_case(case, threads=threads)             # page in
        t1, n1 = best(case, 1)
        tn, nn = best(case, threads)
        t64, n64 = best(case, threads, "f64")
        per[name] = {"workload": desc, "ms_1_thread": round(t1 * 1e3, 3),
                     f"ms_{threads}_threads": round(tn * 1e3, 3),
                     f"ms_f64_{threads}_threads": round(t64 * 1e3, 3),
                     "runs": [n1, nn, n64]}
    head = per["decode16"]
    return {"value": round(head[f"ms_{threads}_threads"] * 1e3, 1), "unit": "us",
            "cores": threads, "kind": "oracle",
            "value_1_thread": round(head["ms_1_thread"] * 1e3, 1),
            "cores_available": {"affinity": host_cores(), "os_cpu_count": os.cpu_count(),
                                "omp_num_threads": os.environ.get("OMP_NUM_THREADS")},
            "cpu_model": host_cpu_model(),
            "sample": f"each of the five workloads run whole, repeated for {seconds:g} s per "
                      f"setting (fastest run kept): fp32 on 1 and on {threads} threads, fp64 on "
                      f"{threads}; value = the decode 16x1 step on {threads} threads; "
                      f"{time.perf_counter() - total_s:.1f} s in all",
            "per_config": per}


def _timed(fn, n, stream):
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def sleep_cycles_per_ms(stream):
    """Clock rate of torch's spin kernel (cycles per ms), measured once."""
    import torch
    torch.cuda._sleep(1000)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(2_000_000)
    b.record(stream)
    torch.cuda.synchronize()
    return 2_000_000 / max(a.elapsed_time(b), 1e-3)


def queued_steps_ms(calls, warmup, stream, cycles_per_ms):
    """``warmup`` untimed calls (calls[i % len]), then exactly len(calls)
    calls timed between two HIP events.  A spin kernel enqueued ahead of the
    start event keeps the GPU busy while the host enqueues the timed calls, so
    they run back to back from the queue: the timed region holds their
    kernels and the gaps between them, not the host's launch cost.  Returns
    (total milliseconds, host enqueue milliseconds, spin milliseconds); the
    host time below the spin time shows that the queue never ran dry."""
    import torch
    if warmup:
        calls[0]()                                   # first launch: loading, set-up
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(1, warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    per_call = (time.perf_counter() - t0) / (warmup - 1) if warmup > 1 else 50e-6
    spin_ms = min(200.0, max(2.0, 3e3 * per_call * len(calls)))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(cycles_per_ms * spin_ms))
    a.record(stream)
    t1 = time.perf_counter()
    for f in calls:
        f()
    host_ms = (time.perf_counter() - t1) * 1e3
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b), host_ms, spin_ms


def calib_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mamba2_selective_scan_amd", "libssmcalib.so"))
    lib.ssm_calib_stream_rw.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    lib.ssm_calib_stream_rw.restype = ctypes.c_int
    return lib


def stream_ceiling(state, n_sets, steps, warmup, stream, cycles_per_ms):
    """The hand-written read-modify-write stream over the same rotated slot
    sets as the decode step (each set: DECODE_SEQS slots, 33.5 MB read and
    written), for 1, 2, 4 and 8 float4 per lane, timed like the decode steps;
    returns the best lane count and the microseconds per launch of each."""
    import ctypes
    lib = calib_lib()
    per_set = DECODE_SEQS * H * P * N            # floats per slot set
    h = ctypes.c_void_p(stream.cuda_stream)
    out = {}
    for pl in (1, 2, 4, 8):
        def call(k, pl=pl):
            rc = lib.ssm_calib_stream_rw(ctypes.c_void_p(state.data_ptr() + 4 * k * per_set),
                                         per_set // 4, pl, 1.0, 0.0, h)
            if rc != 0:
                raise RuntimeError(f"ssm_calib_stream_rw: {rc}")
        calls = [(lambda i=i: call(i % n_sets)) for i in range(steps)]
        out[pl] = 1e3 * queued_steps_ms(calls, warmup, stream, cycles_per_ms)[0] / steps
    pl_best = min(out, key=out.get)
    return pl_best, out


def profile_mode(args, dev, stream):
    """One kernel kind, eager launches, for counter and trace runs: every
    dispatch of the named kernel is the workload of the headline (decode), of
    the prefill (split on the matrix cores, or one pass on the VALU), of the
    chunked gated delta rule, or a plain copy / stream for calibrating
    counters."""
    import torch

    import mamba2_selective_scan_amd as ssm
    import ssm_inputs
    out = {"mode": args.mode}
    if args.mode == "copy":
        n = 256 * 1024 * 1024 // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        ms = _timed(lambda i: dst.copy_(src), args.steps, stream)
        out.update(bytes_read=4 * n, bytes_written=4 * n, ms=ms,
                   GBs=2 * 4 * n / (ms * 1e-3) / 1e9)
    elif args.mode == "stream16":
        state = torch.zeros((DECODE_SEQS * SLOT_SETS, H, P, N), dtype=torch.float32, device=dev)
        cpm = sleep_cycles_per_ms(stream)
        pl, us = stream_ceiling(state, SLOT_SETS, args.steps, args.warmup, stream, cpm)
        nbytes = 2 * 4 * DECODE_SEQS * H * P * N
        out.update(bytes_per_launch=nbytes, us_per_launch=us, best_per_lane=pl,
                   GBs=nbytes / (us[pl] * 1e-6) / 1e9)
    elif args.mode == "decode":
        case = ssm_inputs.workload("decode16", sets=SLOT_SETS)
        d = ssm.to_device(case, dev)
        sets = [torch.arange(k * DECODE_SEQS, (k + 1) * DECODE_SEQS, dtype=torch.int32,
                             device=dev) for k in range(SLOT_SETS)]
        y = torch.empty((DECODE_SEQS, H, P), dtype=torch.float32, device=dev)

        def step(i):
            ssm.decode(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"],
                       sets[i % SLOT_SETS], d["fresh"], y=y)
        for i in range(args.warmup):
            step(i)
        ms = _timed(step, args.steps, stream)
        out.update(algorithmic_bytes=decode_bytes(), ms_per_launch_eager=ms)
    elif args.mode == "gdn_prefill":
        c = ssm_inputs.gdn_workload("prefill4096")
        t = {f: torch.from_numpy(getattr(c, f)).to(dev)
             for f in ("q", "k", "v", "g", "beta", "state", "cu_seqlens", "slot", "fresh")}
        Hv, D = t["v"].shape[1], t["v"].shape[2]
        y = torch.empty((c.n_tokens, Hv, D), device=dev)
        max_len = int((c.cu_seqlens[1:] - c.cu_seqlens[:-1]).max())
        ws = torch.empty(max(ssm.gdn_workspace_size(Hv, t["k"].shape[1], t["k"].shape[2], D,
                                                    int(c.slot.shape[0]), max_len), 1),
                         dtype=torch.uint8, device=dev)

        def once(i):
            ssm.gdn_prefill_ws(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state"],
                               t["cu_seqlens"], t["slot"], t["fresh"], max_len, y=y, workspace=ws)
        for i in range(args.warmup):
            once(i)
        ms = _timed(once, args.steps, stream)
        out.update(algorithmic_flops=7 * c.n_tokens * Hv * D * D, ms_per_launch=ms)
    else:
        pc = ssm_inputs.workload("prefill4096")
        pd = ssm.to_device(pc, dev)
        py = torch.empty((PREFILL_T, H, P), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, ssm.workspace_size(H, P, N, G, 1, PREFILL_T, PREFILL_T)),
                         dtype=torch.uint8, device=dev)

        def once(i):
            if args.mode == "prefill":
                ssm.prefill_ws(pd["x"], pd["dt"], pd["A"], pd["B"], pd["C"], pd["state"],
                               pd["cu_seqlens"], pd["slot"], pd["fresh"], PREFILL_T,
                               workspace=ws, y=py)
            else:
                ssm.prefill(pd["x"], pd["dt"], pd["A"], pd["B"], pd["C"], pd["state"],
                            pd["cu_seqlens"], pd["slot"], pd["fresh"], y=py)
        for i in range(args.warmup):
            once(i)
        ms = _timed(once, args.steps, stream)
        out.update(algorithmic_bytes=prefill_bytes(), algorithmic_flops=prefill_flops(),
                   ms_per_launch=ms)
    out["kernel_hash"] = kernel_source_hash()
    print(json.dumps(out), flush=True)


def summarize_trace(path):
    """Per (kernel, grid size) dispatch statistics from a rocprofv3 kernel
    trace (``*_kernel_trace.csv``): count, median, mean, min and max duration
    in microseconds.  Prints one JSON object (the input of the committed
    kernel-trace summaries under profiles/)."""
    import csv
    import statistics
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("KernelName") or "?"
            grid = r.get("Grid_Size") or r.get("Grid_Size_X") or r.get("Grid_Sizes") or "?"
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            rows.setdefault((name, grid), []).append(dur)
    out = []
    for (name, grid), d in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        out.append({"kernel": name, "grid": grid, "count": len(d),
                    "median_us": round(statistics.median(d), 3),
                    "mean_us": round(statistics.fmean(d), 3), "min_us": round(min(d), 3),
                    "max_us": round(max(d), 3)})
    print(json.dumps({"kernel_hash": kernel_source_hash(), "trace": os.path.basename(path),
                      "kernels": out}, indent=1))


_CPM = None


def _event_ms(fn, n, warm, stream):
    """Milliseconds per call of ``fn``: ``warm`` untimed calls, then ``n``
    calls queued behind a spin kernel and timed between HIP events (so short
    kernels are not padded by the host's launch cost)."""
    global _CPM
    if _CPM is None:
        _CPM = sleep_cycles_per_ms(stream)
    return queued_steps_ms([fn] * n, warm, stream, _CPM)[0] / n


def secondary(args, dev, stream):
    """Time the other workloads and the option paths (eager launches, HIP
    events; each is also a GPU parity case in tests/)."""
    import numpy as np
    import torch

    import mamba2_selective_scan_amd as ssm
    import ssm_inputs
    out = {}
    # decode 256 x 1: 1.07 GB of state traffic per step, far past any cache
    c = ssm_inputs.workload("decode256")
    d = ssm.to_device(c, dev)
    y = torch.empty((256, H, P), device=dev)
    us = 1e3 * _event_ms(lambda: ssm.decode(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"],
                                             d["slot"], d["fresh"], y=y), 20, 3, stream)
    gbs = decode_bytes(256) / (us * 1e-6) / 1e9
    out["decode_256x1"] = {"us": round(us, 2), "GBs": round(gbs, 1),
                           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes": decode_bytes(256)}
    del d, y
    # mixed edge batch, through prefill_ws with its automatic plan (which
    # keeps a batch this short in one pass per sequence)
    c = ssm_inputs.workload("mixed")
    d = ssm.to_device(c, dev)
    ym = torch.empty((c.n_tokens, c.H, c.P), device=dev)
    ml = int(max(c.lengths))
    plan = ssm.prefill_plan(c.H, c.P, c.N, c.G, c.n_seqs, ml)
    wsm = torch.empty(max(ssm.workspace_size(c.H, c.P, c.N, c.G, c.n_seqs, c.n_tokens, ml), 256),
                      dtype=torch.uint8, device=dev)
    us = 1e3 * _event_ms(lambda: ssm.prefill_ws(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"],
                                                 d["cu_seqlens"], d["slot"], d["fresh"], ml,
                                                 workspace=wsm, y=ym),
                         20, 3, stream)
    out["mixed_batch"] = {"us": round(us, 2), "tokens": c.n_tokens, "segments": plan["segments"],
                          "workload": "8 seqs, lengths 1..150, H16 P96 N100 G4"}
    # options on the headline shapes
    pc = ssm_inputs.workload("prefill4096")
    pd = ssm.to_device(pc, dev)
    py = torch.empty((PREFILL_T, H, P), device=dev)
    rng = np.random.Generator(np.random.PCG64(7))
    bias = torch.from_numpy(rng.uniform(-4, 1, H).astype(np.float32)).to(dev)
    ws = torch.empty(max(1, ssm.workspace_size(H, P, N, G, 1, PREFILL_T, PREFILL_T)),
                     dtype=torch.uint8, device=dev)
    base = (pd["x"], pd["dt"], pd["A"], pd["B"], pd["C"], pd["state"], pd["cu_seqlens"],
            pd["slot"], pd["fresh"])
    ms = _event_ms(lambda: ssm.prefill_ws(*base, PREFILL_T, workspace=ws, y=py, dt_bias=bias,
                                          dt_softplus=True), 5, 2, stream)
    out["prefill_1x4096_softplus_bias"] = {"ms": round(ms, 4), "path": "time split"}
    A_hn = torch.from_numpy((-np.exp(rng.uniform(0, np.log(16), (H, N)))).astype(np.float32)).to(dev)
    base_a = (pd["x"], pd["dt"], A_hn) + base[3:]
    ms = _event_ms(lambda: ssm.prefill(*base_a, y=py, A_per_state=True, dt_softplus=True),
                   5, 2, stream)
    out["prefill_1x4096_A_per_state"] = {"ms": round(ms, 4), "path": "whole sequence"}
    short = ssm_inputs.make_case(H, P, N, G, [8] * 16, [0] * 16, seed=8)
    sd = ssm.to_device(short, dev)
    snaps = torch.empty((short.n_tokens, H, P, N), device=dev)
    ys = torch.empty((short.n_tokens, H, P), device=dev)
    us = 1e3 * _event_ms(lambda: ssm.prefill(sd["x"], sd["dt"], sd["A"], sd["B"], sd["C"],
                                              sd["state"], sd["cu_seqlens"], sd["slot"],
                                              sd["fresh"], y=ys, snapshots=snaps), 20, 3, stream)
    out["draft_16x8_snapshots"] = {"us": round(us, 2),
                                   "workload": "16 seqs x 8 draft tokens, state after every token "
                                               "written (268 MB of snapshots)"}
    dd = ssm.to_device(ssm_inputs.workload("decode16"), dev)
    yd = torch.empty((16, H, P), device=dev)
    us = 1e3 * _event_ms(lambda: ssm.decode(dd["x"], dd["dt"], dd["A"], dd["B"], dd["C"],
                                             dd["state"], dd["slot"], dd["fresh"], y=yd,
                                             dt_bias=bias, dt_softplus=True), 50, 5, stream)
    out["decode_16x1_softplus_bias_eager"] = {"us": round(us, 2),
                                              "note": "eager launches, one slot set (warm cache)"}
    return out


def _graph_us(calls, replays, stream):
    """Capture ``calls`` (closures that each enqueue one launch) in one HIP
    graph, replay it ``replays`` times between HIP events and return the
    average time per call in microseconds (launch overhead out of the way)."""
    import torch
    for f in calls:                                     # eager warm-up
        f()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for f in calls:
            f()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (replays * len(calls))


def beside(args, dev, stream):
    """The steps beside the scan in a layer at the same geometry: causal conv1d
    + SiLU over D = H*P + 2*G*N channels (K = 4) and gated RMSNorm over y
    [T][H][P].  Both are HBM-bound; algorithmic bytes count every operand
    once (the conv history only where it is read or written).  Each line is
    the average over a replayed HIP graph of 8 launches."""
    import torch

    import mamba2_selective_scan_amd as ssm
    import ssm_inputs
    out = {}
    D = ssm_inputs.conv_channels(H, P, N, G)
    K = 4

    def line(us, nbytes, **extra):
        gbs = nbytes / (us * 1e-6) / 1e9
        return dict({"us": round(us, 2), "GBs": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes},
                    **extra)

    c = ssm_inputs.conv_workload("prefill4096")
    t = {f: torch.from_numpy(getattr(c, f)).to(dev)
         for f in ("x", "w", "state", "cu_seqlens", "slot", "fresh")}
    o = torch.empty((PREFILL_T, D), device=dev)
    conv = lambda: ssm.conv1d_silu(t["x"], t["w"], t["state"], t["cu_seqlens"], t["slot"],
                                   t["fresh"], out=o)
    us = _graph_us([conv] * 8, 10, stream)
    nbytes = 4 * (2 * PREFILL_T * D + D * K + D * (K - 1))
    out["conv1d_silu_prefill_1x4096_D6144_K4"] = line(us, nbytes)
    del t, o
    # decode: rotate over 8 slot sets so the histories are not cache-resident
    for n_seq in (16, 256):
        sets = 8
        c = ssm_inputs.make_conv_case(D, K, [1] * n_seq, [0] * n_seq, 11, n_slots=n_seq * sets)
        x, w = torch.from_numpy(c.x).to(dev), torch.from_numpy(c.w).to(dev)
        st = torch.from_numpy(c.state).to(dev)
        fresh = torch.from_numpy(c.fresh).to(dev)
        slots = [torch.arange(k * n_seq, (k + 1) * n_seq, dtype=torch.int32, device=dev)
                 for k in range(sets)]
        o = torch.empty((n_seq, D), device=dev)
        calls = [(lambda k=k: ssm.conv1d_silu_decode(x, w, st, slots[k], fresh, out=o))
                 for k in range(sets)]
        us = _graph_us(calls, 40, stream)
        nbytes = 4 * (2 * n_seq * D + D * K + 2 * n_seq * D * (K - 1))
        out[f"conv1d_silu_decode_{n_seq}x1_D6144_K4"] = line(
            us, nbytes, note=f"{sets} history slot sets rotated")
        del x, w, st, o, slots, calls
    for name, T in (("prefill4096", PREFILL_T), ("decode16", 16), ("decode256", 256)):
        nc = ssm_inputs.norm_workload(name)
        y, z, w = (torch.from_numpy(getattr(nc, f)).to(dev) for f in ("y", "z", "w"))
        o = torch.empty_like(y)
        us = _graph_us([lambda: ssm.gated_rmsnorm(y, z, w, nc.eps, out=o)] * 8, 20, stream)
        nbytes = 4 * (3 * T * H * P + P)
        out[f"gated_rmsnorm_{T}x{H}x{P}"] = line(us, nbytes)
    return out


def gated_delta(args, dev, stream):
    """The gated delta-rule recurrence at the page's model geometry (Hv 32,
    Hk 16, Dk = Dv = 128): prefill 1 x 4096 (algorithmic work 7 flop per state
    value per token: decay, the two dots, the write), timed in the chunked
    matrix form (``gdn_prefill_ws``, workspace allocated once outside the timed
    calls) and, as context, in the per-token VALU kernel (``gdn_prefill``); and
    decode 16 x 1 / 256 x 1 (HBM-bound; the state read and written once).
    Decode 16 rotates 16 slot sets through a replayed HIP graph, as the
    scan's."""
    import torch

    import mamba2_selective_scan_amd as ssm
    import ssm_inputs
    out = {}
    Hv, Hk, D = 32, 16, 128
    c = ssm_inputs.gdn_workload("prefill4096")
    t = {f: torch.from_numpy(getattr(c, f)).to(dev)
         for f in ("q", "k", "v", "g", "beta", "state", "cu_seqlens", "slot", "fresh")}
    y = torch.empty((c.n_tokens, Hv, D), device=dev)
    max_len = int((c.cu_seqlens[1:] - c.cu_seqlens[:-1]).max())
    n_seqs = int(c.slot.shape[0])
    ws = torch.empty(max(ssm.gdn_workspace_size(Hv, Hk, D, D, n_seqs, max_len), 1),
                     dtype=torch.uint8, device=dev)
    flops = 7 * PREFILL_T * Hv * D * D
    ms_c = _event_ms(lambda: ssm.gdn_prefill_ws(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                t["state"], t["cu_seqlens"], t["slot"],
                                                t["fresh"], max_len, y=y, workspace=ws),
                     10, 3, stream)
    ms = _event_ms(lambda: ssm.gdn_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state"],
                                           t["cu_seqlens"], t["slot"], t["fresh"], y=y), 10, 3, stream)
    tf_c = flops / (ms_c * 1e-3) / 1e12
    tf = flops / (ms * 1e-3) / 1e12
    out["gdn_prefill_1x4096_Hv32_Hk16_D128"] = {
        "ms": round(ms_c, 4), "entry": "ssm_gdn_prefill_ws (chunks of 32 tokens, matrix cores)",
        "TFLOPs": round(tf_c, 2), "frac_fp32_mfma": round(tf_c / FP32_MFMA_PEAK_TFLOPS, 4),
        "workspace_bytes": int(ws.numel()), "algorithmic_flops": flops,
        "per_token_kernel": {
            "ms": round(ms, 4), "entry": "ssm_gdn_prefill", "TFLOPs": round(tf, 2),
            "frac_fp32": round(tf / FP32_VALU_PEAK_TFLOPS, 4),
            "frac_unpacked_fp32": round(tf / FP32_VALU_UNPACKED_TFLOPS, 4)}}
    del t, y, ws

    def dec_bytes(n):
        return 4 * (2 * n * Hv * D * D + n * (2 * Hk * D + 2 * Hv * D + 2 * Hv))

    for n_seq, sets in ((16, 16), (256, 1)):
        c = ssm_inputs.make_gdn_case(Hv, Hk, D, D, [1] * n_seq, [0] * n_seq, 31,
                                     n_slots=n_seq * sets)
        t = {f: torch.from_numpy(getattr(c, f)).to(dev)
             for f in ("q", "k", "v", "g", "beta", "state", "fresh")}
        slots = [torch.arange(k * n_seq, (k + 1) * n_seq, dtype=torch.int32, device=dev)
                 for k in range(sets)]
        y = torch.empty((n_seq, Hv, D), device=dev)
        calls = [(lambda k=k: ssm.gdn_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state"],
                                             slots[k], t["fresh"], y=y)) for k in range(sets)]
        us = _graph_us(calls, max(2, 320 // sets), stream)
        gbs = dec_bytes(n_seq) / (us * 1e-6) / 1e9
        out[f"gdn_decode_{n_seq}x1_Hv32_Hk16_D128"] = {
            "us": round(us, 2), "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": dec_bytes(n_seq), "slot_sets_rotated": sets}
        del t, y, slots, calls
    return out


def summarize_counters(path):
    """Per-kernel means of each counter in a rocprofv3 counter collection
    (``*_counter_collection.csv``), over that kernel's dispatches.  Prints one
    JSON object (the input of the committed counter summaries)."""
    import csv
    import statistics
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"]
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {k: {c: {"mean": statistics.fmean(v), "dispatches": len(v)} for c, v in cs.items()}
           for k, cs in acc.items()}
    print(json.dumps({"kernel_hash": kernel_source_hash(), "counters": os.path.basename(path),
                      "kernels": out}, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=32, help="untimed decode steps")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=1.0,
                    help="oracle timing budget per workload and setting")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary workloads (decode 256x1, mixed batch, options)")
    ap.add_argument("--mode", choices=("all", "decode", "prefill", "prefill1", "gdn_prefill", "copy",
                                       "stream16"),
                    default="all",
                    help="decode/prefill: launch only that path (prefill: the time-split path; "
                         "prefill1: the unsplit single kernel; gdn_prefill: the chunked "
                         "gated delta rule, 1 x 4096), eagerly, and print its "
                         "timing (for counter runs); copy: a plain 256 MiB device copy, the "
                         "reference for scaling HBM byte counters; stream16: the read-modify-"
                         "write stream over the decode step's 16 rotating slot sets")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print per-kernel statistics of a rocprofv3 kernel trace and exit")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="print per-kernel counter means of a rocprofv3 counter collection and exit")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the scan needs no collective and this build runs "
              "on a single MI355X (see the sharding notes); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mamba2_selective_scan_amd as ssm
    import ssm_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.mode != "all":
        profile_mode(args, dev, stream)
        return
    cpm = sleep_cycles_per_ms(stream)

    # ---------------- decode 16x1, 16 rotating slot sets
    case = ssm_inputs.workload("decode16", sets=SLOT_SETS)
    d = ssm.to_device(case, dev)
    slot_sets = [torch.arange(k * DECODE_SEQS, (k + 1) * DECODE_SEQS, dtype=torch.int32,
                              device=dev) for k in range(SLOT_SETS)]
    y = torch.empty((DECODE_SEQS, H, P), dtype=torch.float32, device=dev)

    def decode_step(k):
        ssm.decode(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"], slot_sets[k],
                   d["fresh"], y=y)

    calls = [(lambda i=i: decode_step(i % SLOT_SETS)) for i in range(args.steps)]
    t0 = time.perf_counter()
    dec_ms, host_ms, spin_ms = queued_steps_ms(calls, args.warmup, stream, cpm)
    wall = time.perf_counter() - t0
    dec_us = dec_ms * 1e3 / args.steps                   # average step (= launch) duration
    dec_gbs = decode_bytes() / (dec_us * 1e-6) / 1e9
    # the ceiling: a plain read-modify-write stream over the same slot sets
    pl, st_us = stream_ceiling(d["state"], SLOT_SETS, args.steps, args.warmup, stream, cpm)
    st_gbs = 2 * 4 * DECODE_SEQS * H * P * N / (st_us[pl] * 1e-6) / 1e9
    trace = load_profile("decode16_kernel_trace")

    result = {
        "metric": "scan time per layer (ms prefill 1x4096, us decode 16x1); % HBM/VALU roofline",
        "value": round(dec_us, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec_us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; x,B,C ~ N(0,1), dt ~ U[0.001,0.1], A = -exp(U[0,ln16]), "
                "state ~ 0.5 N(0,1))",
        "config": {"workload": "decode 16 seqs x 1 token, resuming", "H": H, "P": P, "N": N,
                   "G": G, "slot_sets_rotated": SLOT_SETS,
                   "state_bytes_rotated": int(case.state.nbytes),
                   "launch": f"{args.warmup} untimed steps, then {args.steps} steps queued "
                             "behind a spin kernel and timed between HIP events",
                   "host_enqueue_ms": round(host_ms, 3), "spin_ms": round(spin_ms, 3),
                   "geometry": ssm.geometry(H, P, N, G, DECODE_SEQS, decode=True)},
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("decode16"),
                     "algorithmic_bytes_per_launch": decode_bytes(),
                     "achievable": {"kernel": "read-modify-write stream over the same slot "
                                              f"sets ({pl} float4 per lane, best of 1/2/4/8)",
                                    "us": round(st_us[pl], 3), "GBs": round(st_gbs, 1),
                                    "us_per_lane_count": {str(k): round(v, 3)
                                                          for k, v in st_us.items()},
                                    "frac_of_achievable": round(st_us[pl] / dec_us, 4)},
                     "kernel_trace": None if trace is None else {
                         "median_us": trace.get("median_us"), "mean_us": trace.get("mean_us"),
                         "source": trace.get("source")}},
        "wall_s_timed": round(wall, 4),
        "timed_steps_ms": round(dec_ms, 4),
    }

    # ---------------- prefill 1x4096, fresh.  On the matrix cores: the library
    # splits the one sequence over time (ssm_scan_prefill_ws, automatic plan).
    # On the VALU: the one-pass register kernel (ssm_scan_prefill).
    if not args.no_prefill:
        pc = ssm_inputs.workload("prefill4096")
        pd = ssm.to_device(pc, dev)
        py = torch.empty((PREFILL_T, H, P), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, ssm.workspace_size(H, P, N, G, 1, PREFILL_T, PREFILL_T)),
                         dtype=torch.uint8, device=dev)

        def prefill_split():
            ssm.prefill_ws(pd["x"], pd["dt"], pd["A"], pd["B"], pd["C"], pd["state"],
                           pd["cu_seqlens"], pd["slot"], pd["fresh"], PREFILL_T,
                           workspace=ws, y=py)

        def prefill_unsplit():
            ssm.prefill(pd["x"], pd["dt"], pd["A"], pd["B"], pd["C"], pd["state"],
                        pd["cu_seqlens"], pd["slot"], pd["fresh"], y=py)

        def event_times(fn):
            for _ in range(args.prefill_warmup):
                fn()
            torch.cuda.synchronize()
            pairs = []
            for _ in range(args.prefill_steps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                pairs.append((a, b))
            torch.cuda.synchronize()
            return [a.elapsed_time(b) for a, b in pairs]

        def stats(ms):
            return {"ms": round(float(np.mean(ms)), 4), "ms_median": round(float(np.median(ms)), 4),
                    "ms_min": round(min(ms), 4), "ms_max": round(max(ms), 4),
                    "iterations": args.prefill_steps, "warmup": args.prefill_warmup}

        ms = event_times(prefill_split)
        ms1 = event_times(prefill_unsplit)
        pf_ms, pf1_ms = float(np.mean(ms)), float(np.mean(ms1))
        tflops = prefill_flops() / (pf_ms * 1e-3) / 1e12
        tflops1 = prefill_flops() / (pf1_ms * 1e-3) / 1e12
        counters = load_profile("prefill4096_counters") or {}
        result["prefill"] = dict(stats(ms), **{
            "workload": "prefill 1 seq x 4096 tokens, fresh",
            "path": "ssm_scan_prefill_ws, automatic time split: matrix-core state pass (end "
                    "states of segments 0..n-2), carry combine, matrix-core chunked scans of every "
                    "segment from its carried-in state (3 kernels)",
            "plan": ssm.prefill_plan(H, P, N, G, 1, PREFILL_T),
            # the dominant kernels are fp32 matrix-core contractions; MI355X's
            # dense fp32 MFMA peak is the same 157.3 TFLOP/s as its packed vector
            # peak.  `achieved` counts the recurrence's own 5 flop per state
            # element per token (the chunked form does more arithmetic).
            "roofline": {"bound": "mfma", "achieved": round(tflops, 3),
                         "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4),
                         "traffic": load_traffic("prefill4096"),
                         "algorithmic_flops_per_launch": prefill_flops(),
                         "algorithmic_bytes_per_launch": prefill_bytes(),
                         "achieved_GBs": round(prefill_bytes() / (pf_ms * 1e-3) / 1e9, 1)},
            "counters": counters.get("split"),
        })
        geo1 = ssm.geometry(H, P, N, G, 1)
        result["prefill_valu"] = dict(stats(ms1), **{
            "workload": "prefill 1 seq x 4096 tokens, fresh",
            "path": f"ssm_scan_prefill: one pass per (head, {geo1['rows_per_block']}-row block), "
                    f"state in registers ({geo1['lanes_per_row']} lanes x {geo1['elems_per_lane']} "
                    f"per row), y by DPP reduce-scatter, chunks of {geo1['chunk_tokens']} tokens "
                    "staged in LDS (the VALU path)",
            "geometry": geo1,
            "roofline": {"bound": "alu", "achieved": round(tflops1, 3),
                         "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops1 / FP32_VALU_PEAK_TFLOPS, 4),
                         "frac_of_unpacked_fp32": round(tflops1 / FP32_VALU_UNPACKED_TFLOPS, 4),
                         "traffic": None,
                         "algorithmic_flops_per_launch": prefill_flops()},
            "counters": counters.get("valu"),
        })

    if not args.no_secondary:
        result["secondary"] = secondary(args, dev, stream)
        result["beside_the_scan"] = beside(args, dev, stream)
        result["gated_delta_rule"] = gated_delta(args, dev, stream)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    result["device"] = torch.cuda.get_device_name(dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
