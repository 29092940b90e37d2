#!/usr/bin/env python3
"""Benchmark of the MI355X Mamba2 selective-state scan (one layer's scan).

Headline: decode, 16 sequences x 1 token at H=64, P=64, N=128, G=8, fp32,
resuming state.  A step is one ssm_scan_decode call.  Consecutive steps use
16 disjoint slot sets of a 256-slot state (537 MB), so each step's 33.5 MB of
state comes from HBM, not from the 256 MB Infinity Cache.  The 16 steps of one
rotation are captured once in a HIP graph and replayed, so host launch
overhead does not pad the step time.  Also measured and reported beside it:
the 1 x 4096-token prefill at the same geometry (fresh state, eager launches,
the automatic time split on the matrix cores), the secondary scan workloads,
the ops beside the scan (conv1d + SiLU, gated RMSNorm) and the gated delta rule.

Prints one JSON line.  Times come from HIP events on the stream the kernels run
on; the roofline objects use algorithmic bytes (decode, HBM-bound) and
algorithmic flops (prefill, bound by the FP32 matrix cores).
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


def load_traffic(name):
    """Measured HBM bytes per launch from a committed counter run, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


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


def cpu_baseline_decode(case, seconds):
    """The fp32 oracle on the same decode step, repeated for ~``seconds`` on
    all host threads (up to 16) and for ~seconds/3 on one thread."""
    import oracle
    threads = min(16, host_cores())
    orc = oracle.default()

    def rate(th, budget):
        orc.scan_case(case, threads=th)                # page in
        n, t0 = 0, time.perf_counter()
        while True:
            orc.scan_case(case, threads=th)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return n, el
    n, el = rate(threads, seconds)
    n1, el1 = rate(1, max(1.0, seconds / 3))
    return {"value": round(el / n * 1e6, 1), "unit": "us", "cores": threads, "kind": "oracle",
            "value_1_thread": round(el1 / n1 * 1e6, 1), "cpu_model": host_cpu_model(),
            "sample": f"{n} repetitions of the full decode 16x1 step (16 seqs x 64 heads x 64 "
                      f"rows x 128 state, fp32, resuming) on {threads} threads, {el:.1f} s; "
                      f"{n1} on 1 thread, {el1:.1f} s"}


def _timed(fn, n, stream):
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def profile_mode(args, dev, stream):
    """One kernel kind, eager launches, for counter runs: every dispatch of the
    named kernel is the workload of the headline (decode) or of the prefill."""
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
    elif args.mode == "copy16":
        n = DECODE_SEQS * H * P * N
        src = [torch.randn(n, device=dev) for _ in range(SLOT_SETS)]
        dst = [torch.empty_like(src[0]) for _ in range(SLOT_SETS)]

        def rot():
            for k in range(SLOT_SETS):
                dst[k].copy_(src[k])
        rot()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            rot()
        for _ in range(2):
            graph.replay()
        ms = _timed(lambda i: graph.replay(), max(1, args.steps // SLOT_SETS), stream) / SLOT_SETS
        out.update(bytes_per_copy=2 * 4 * n, us_per_copy=ms * 1e3,
                   GBs=2 * 4 * n / (ms * 1e-3) / 1e9)
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


def _event_ms(fn, n, warm, stream):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


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
    # mixed edge batch
    c = ssm_inputs.workload("mixed")
    d = ssm.to_device(c, dev)
    ym = torch.empty((c.n_tokens, c.H, c.P), device=dev)
    us = 1e3 * _event_ms(lambda: ssm.prefill(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"],
                                              d["cu_seqlens"], d["slot"], d["fresh"], y=ym),
                         20, 3, stream)
    out["mixed_batch"] = {"us": round(us, 2), "tokens": c.n_tokens,
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
        "ms": round(ms_c, 4), "entry": "ssm_gdn_prefill_ws (chunks of 16 tokens, matrix cores)",
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=32, help="untimed decode steps")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary workloads (decode 256x1, mixed batch, options)")
    ap.add_argument("--mode", choices=("all", "decode", "prefill", "prefill1", "copy", "copy16"),
                    default="all",
                    help="decode/prefill: launch only that path (prefill: the time-split path; "
                         "prefill1: the unsplit single kernel), eagerly, and print its "
                         "timing (for counter runs); copy: a plain 256 MiB device copy, the "
                         "reference for scaling HBM byte counters; copy16: device copies of "
                         "one decode step's state size over 16 rotating buffers, replayed "
                         "from a HIP graph like the decode bench (achievable-bandwidth "
                         "reference)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the scan needs no collective and this build runs "
              "on a single MI355X (see the sharding notes); run it with --gpus 1.",
              file=sys.stderr)
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

    # ---------------- decode 16x1, 16 rotating slot sets
    case = ssm_inputs.workload("decode16", sets=SLOT_SETS)
    d = ssm.to_device(case, dev)
    slot_sets = [torch.arange(k * DECODE_SEQS, (k + 1) * DECODE_SEQS, dtype=torch.int32,
                              device=dev) for k in range(SLOT_SETS)]
    y = torch.empty((DECODE_SEQS, H, P), dtype=torch.float32, device=dev)

    def decode_step(k):
        ssm.decode(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"], slot_sets[k],
                   d["fresh"], y=y)

    for k in range(SLOT_SETS):                          # eager warm-up, sets the kernels up
        decode_step(k)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(SLOT_SETS):
            decode_step(k)
    torch.cuda.synchronize()
    replays_w = max(1, -(-args.warmup // SLOT_SETS))
    replays = max(1, -(-args.steps // SLOT_SETS))
    steps = replays * SLOT_SETS
    for _ in range(replays_w):
        graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(replays):
        graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_us = ev0.elapsed_time(ev1) * 1e3 / steps        # average step (= launch) duration
    dec_gbs = decode_bytes() / (dec_us * 1e-6) / 1e9
    traffic = load_traffic("decode16")

    result = {
        "metric": "scan time per layer (ms prefill 1x4096, us decode 16x1); % HBM/VALU roofline",
        "value": round(dec_us, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": steps,
        "warmup": replays_w * SLOT_SETS,
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
                   "launch": "HIP graph of 16 steps, replayed",
                   "geometry": ssm.geometry(H, P, N, G, DECODE_SEQS, decode=True)},
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": decode_bytes()},
        "wall_s_timed": round(wall, 4),
    }

    # ---------------- prefill 1x4096, fresh.  One sequence fills only a quarter
    # of the SIMDs, so the library splits it over time (ssm_scan_prefill_ws,
    # automatic plan); the unsplit single-pass time is reported beside it.
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

        ms = event_times(prefill_split)
        ms_unsplit = event_times(prefill_unsplit)
        pf_ms = float(np.mean(ms))
        tflops = prefill_flops() / (pf_ms * 1e-3) / 1e12
        result["prefill"] = {
            "workload": "prefill 1 seq x 4096 tokens, fresh", "ms": round(pf_ms, 4),
            "ms_min": round(min(ms), 4), "ms_max": round(max(ms), 4),
            "iterations": args.prefill_steps,
            "path": "ssm_scan_prefill_ws, automatic time split: matrix-core state pass (end "
                    "states of segments 0..n-2), carry combine, matrix-core chunked scans of every "
                    "segment from its carried-in state, two 16-row tiles per wave (3 kernels)",
            "plan": ssm.prefill_plan(H, P, N, G, 1, PREFILL_T),
            "ms_unsplit": round(float(np.mean(ms_unsplit)), 4),
            "geometry_unsplit": ssm.geometry(H, P, N, G, 1),
            # both dominant kernels are fp32 matrix-core contractions now; MI355X's
            # dense fp32 MFMA peak is the same 157.3 TFLOP/s as its packed vector
            # peak.  `achieved` counts the recurrence's own 5 flop per state
            # element per token (the chunked form does more arithmetic).
            "roofline": {"bound": "mfma", "achieved": round(tflops, 3),
                         "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4),
                         "frac_of_unpacked_fp32": round(tflops / FP32_VALU_UNPACKED_TFLOPS, 4),
                         "traffic": load_traffic("prefill4096"),
                         "algorithmic_flops_per_launch": prefill_flops(),
                         "algorithmic_bytes_per_launch": prefill_bytes(),
                         "achieved_GBs": round(prefill_bytes() / (pf_ms * 1e-3) / 1e9, 1)},
        }

    if not args.no_secondary:
        result["secondary"] = secondary(args, dev, stream)
        result["beside_the_scan"] = beside(args, dev, stream)
        result["gated_delta_rule"] = gated_delta(args, dev, stream)

    if not args.no_cpu_baseline:
        one_set = ssm_inputs.workload("decode16")
        result["cpu_baseline"] = cpu_baseline_decode(one_set, args.cpu_seconds)
    result["device"] = torch.cuda.get_device_name(dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
