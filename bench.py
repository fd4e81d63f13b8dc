#!/usr/bin/env python3
"""Throughput of the selective-SSM scan forward pass on one MI355X.

One step = one ssm_scan_fwd over the Mamba-1.4B-shaped layer (B=4, L=8192,
D=4096, N=16, bf16 x/delta/z/B/C/y, fp32 state, SiLU gate, final state
returned), inputs resident in HBM.  Prints one JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

With a chunked workload (the 256K-token sequence run as 32 chained calls) a
step is the whole chain; with the decode workload a step is its 128
single-token steps.  Those lines add per-call / per-decode-step times.

Before the W warmup steps, every line runs its step untimed for --settle-ms
(300 ms) of wall time: the GPU raises its clocks over the first tens of
milliseconds of sustained load, and a short run would otherwise time the ramp.
The JSON line reports what that phase ran ("settle").

The metric is scan elements per second, B*L*D*N / step time, in GElem/s.  The
roofline object reports the algorithmic HBM bytes of one launch (every input
read once, y and hT written once) over the launch's average duration, timed
with HIP events on the stream the kernel runs on, against the MI355X peak of
8 TB/s.  The CPU baseline times the fp64 oracle on a bounded slice of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# What the clock-settling phase did (added to the JSON line as "settle").
SETTLE = {}


def settle(fn, torch, args):
    """Run fn(i) back to back, untimed, for args.settle_ms of wall time before
    the warmup steps.  Under this sustained load the GPU raises its clocks over
    the first tens of milliseconds: with 5 warmup steps of the 1.4B-shaped
    layer (2.5 ms) the timed launches averaged 498 us, after 100 warmup steps
    403 us, so without this phase a short run times the clock's ramp rather
    than the kernel."""
    if args.settle_ms <= 0:
        return
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(2):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    SETTLE.update({"ms": round((time.perf_counter() - t0) * 1e3, 1), "calls": n})
    log(f"clocks settled: {n} untimed calls in {SETTLE['ms']} ms")


def emit(out):
    if SETTLE:
        out["settle"] = dict(SETTLE, note="untimed calls of the same step before the warmup steps, while the "
                                          "GPU's clocks ramp up under load")
    print(json.dumps(out), flush=True)


def algorithmic_bytes(w) -> int:
    """Bytes one call must move at minimum: x, delta, z read and y written
    (B,L,D each), B and C read (B,L,N), A (D,N), D and delta_bias (D) read,
    h0 read / hT written (B,D,N fp32) where the workload uses them."""
    es = 2 if "bfloat16" in str(w.dtype) else 4
    L = w.seqlen if not w.steps else 1
    bld = w.batch * L * w.dim
    bln = w.batch * L * w.dstate
    n = (3 if w.gate else 2) * bld * es + bld * es  # x, delta, (z) in; y out
    n += 2 * bln * es + w.dim * w.dstate * 4 + 2 * w.dim * 4
    if w.final_state:
        n += w.batch * w.dim * w.dstate * 4
    if w.h0_std > 0:
        n += w.batch * w.dim * w.dstate * 4
    return n


# Sources the forward scan kernels are built from (the backward's are not).
FORWARD_SOURCES = ("buffer_io.hpp", "device_common.hpp", "nsplit_dispatch.cpp", "nsplit_inst.hip",
                   "scan_decode.hip", "scan_lane.hip", "scan_nsplit_impl.hpp")


# the sources of the chunked matrix-form kernel (SSD and gated attention lines)
SSD_SOURCES = ("buffer_io.hpp", "device_common.hpp", "ssd_fwd.hip")
# the sources of the backward kernels (with the forward's, whose checkpoints they read)
BACKWARD_SOURCES = FORWARD_SOURCES + ("scan_bwd.hip", "scan_bwd_impl.hpp", "scan_bwd_inst.hip")


def kernel_source_hash(sources=FORWARD_SOURCES) -> str:
    """Hash of the kernels' HIP sources, so stored traffic counters can be
    matched to the kernel build they were measured on."""
    csrc = os.path.join(HERE, "mamba_selective_scan_06_amd", "csrc")
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload_name: str, sources=FORWARD_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None.  The summary is a text
    file of `key: value` lines."""
    path = os.path.join(HERE, "profiles", f"traffic_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    try:
        return int(rec["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_info():
    """(logical CPUs of the host, CPU model name from /proc/cpuinfo or None)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count() or 1, model


def _slice_channels(inp, nd):
    """The first nd channels of every batch row and token (chains are independent)."""
    out = dict(inp)
    for k in ("x", "delta", "z"):
        if out.get(k) is not None:
            out[k] = out[k][:, :, :nd].contiguous()
    out["A"] = out["A"][:nd].contiguous()
    for k in ("D", "delta_bias"):
        if out.get(k) is not None:
            out[k] = out[k][:nd].contiguous()
    if out.get("h0") is not None:
        out["h0"] = out["h0"][:, :nd].contiguous()
    return out


def cpu_baseline(w, inp, max_threads=16, zoh=False, what="the whole workload"):
    """The fp64 oracle timed on the host: over all of `inp` (the whole workload)
    on all usable cores (at most the 16 of a one-GPU share), and over a channel
    slice on one thread; only the C calls are timed.  `value` is the all-cores
    rate."""
    import oracle
    nproc, model = cpu_info()
    threads = max(1, min(nproc, max_threads))
    B_, L_, D_ = inp["x"].shape
    N_ = inp["A"].shape[1]
    timing = {}
    oracle.scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                inp.get("h0"), threads=threads, timing=timing, zoh=zoh)
    elems = B_ * L_ * D_ * N_
    # one thread: the first channels of every row and token, about 1/16 of the work
    nd = max(1, min(D_, D_ // 16))
    sub = _slice_channels(inp, nd)
    t1 = {}
    oracle.scan(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], sub["delta_bias"],
                sub.get("h0"), threads=1, timing=t1, zoh=zoh)
    el1 = B_ * L_ * nd * N_
    return {
        "value": round(elems / timing["seconds"] / 1e9, 4),
        "unit": "GElem/s",
        "cores": timing["threads"],
        "kind": "oracle",
        "sample": f"{what} (B={B_} L={L_} D={D_} N={N_}, {elems} elements), inputs widened to fp64 "
                  f"beforehand; {timing['seconds']:.2f} s on {timing['threads']} threads",
        "single_thread_value": round(el1 / t1["seconds"] / 1e9, 4),
        "single_thread_sample": f"channels 0..{nd - 1} of every row and token ({el1} elements), "
                                f"{t1['seconds']:.2f} s on 1 thread",
        "nproc": nproc,
        "cpu_model": model,
    }


def io_dtype(w) -> str:
    return "bf16" if "bfloat16" in str(w.dtype) else "f32"


def _roofline(alg_bytes, kern_s, kernel):
    achieved = alg_bytes / kern_s / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kernel,
            "kernel_avg_us": round(kern_s * 1e6, 2), "algorithmic_bytes": alg_bytes}


def bench_chunked(w, args, ssm, torch):
    """A long sequence run as `w.chunks` calls, each starting from the previous
    call's final state (state buffers alternate, so calls may split time).
    One step = all the calls over the whole sequence."""
    import workloads
    dev = torch.device("cuda:0")
    log(f"workload {w.describe()}")
    inp = workloads.make_inputs(w)
    Lc = w.seqlen // w.chunks
    chunks = []
    for c in range(w.chunks):
        sl = slice(c * Lc, (c + 1) * Lc)
        chunks.append({k: (inp[k][:, sl].contiguous().to(dev) if inp[k] is not None else None)
                       for k in ("x", "delta", "z", "B", "C")})
    A, D, bias = (inp[k].to(dev) for k in ("A", "D", "delta_bias"))
    ys = [torch.empty_like(ch["x"]) for ch in chunks]
    hs = [torch.zeros(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream(dev)

    def one_pass(events=None):
        hs[0].zero_()
        for c, ch in enumerate(chunks):
            h_in, h_out = hs[c % 2], hs[(c + 1) % 2]
            if events is not None:
                events[c][0].record(stream)
            ssm.scan_fwd(ch["x"], ch["delta"], A, ch["B"], ch["C"], D, ch["z"], bias,
                         h_in if c > 0 else None, out=ys[c], final_state_out=h_out, time_splits=args.time_splits,
                         carry_scan=args.carry_scan)
            if events is not None:
                events[c][1].record(stream)

    settle(lambda i: one_pass(), torch, args)
    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in chunks] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        one_pass(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_ms = [a.elapsed_time(b) for e in evs for a, b in e]
    per_call_s = float(np.mean(call_ms)) * 1e-3
    es = 2 if "bfloat16" in str(w.dtype) else 4
    bld, bln = w.batch * Lc * w.dim, w.batch * Lc * w.dstate
    state = w.batch * w.dim * w.dstate * 4
    call_bytes = (4 if w.gate else 3) * bld * es + 2 * bln * es + w.dim * w.dstate * 4 + 2 * w.dim * 4 + 2 * state
    probe = ssm.make_args(chunks[1]["x"], chunks[1]["delta"], A, chunks[1]["B"], chunks[1]["C"], D,
                          chunks[1]["z"], bias, hs[0], hs[1], ys[1], None, "auto", args.time_splits)
    nbytes = ssm.workspace_bytes(probe)
    if nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        probe.workspace, probe.workspace_bytes = ws.data_ptr(), nbytes
    plan = ssm.plan(probe)
    ms_per_step = elapsed * 1e3 / steps
    out = {
        "metric": "scan GElem/s (B*L*D*N) over the chained calls + % HBM roofline per call",
        "value": round(w.elems / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GElem/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": io_dtype(w), "state_dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim, "dstate": w.dstate,
                   "io_dtype": str(w.dtype).replace("torch.", ""), "gate": w.gate, "calls": w.chunks,
                   "call_seqlen": Lc, "plan": {"variant": plan[0], "time_splits": plan[1],
                                               "carry": "scan" if args.carry_scan else "serial fold"}},
        "per_call_us": round(per_call_s * 1e6, 2),
        "calls_total_kernel_us": round(per_call_s * w.chunks * 1e6, 2),
        "roofline": _roofline(call_bytes, per_call_s, "scan_nsplit_kernel (+ state-only pass)"),
    }
    out["roofline"]["traffic"] = stored_traffic(w.name)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle over the whole sequence) ...")
        out["cpu_baseline"] = cpu_baseline(
            w, inp, what=f"the whole {w.seqlen}-token sequence as one oracle run (bitwise equal to the "
                         f"{w.chunks} chained oracle calls)")
    return out


def bench_decode(w, args, ssm, torch):
    """`w.steps` successive single-token steps, updating one fp32 state in place
    (fresh inputs each step, generated and moved to the device beforehand).
    One bench step = all the decode steps."""
    import workloads
    dev = torch.device("cuda:0")
    log(f"workload {w.describe()}")
    inp = workloads.make_inputs(w, seqlen=1)
    A, D, bias = (inp[k].to(dev) for k in ("A", "D", "delta_bias"))
    h = inp["h0"].to(dev)
    steps_in = []
    for t in range(w.steps):
        st = workloads.make_decode_step(w, t)
        steps_in.append({k: (v.to(dev) if v is not None else None) for k, v in st.items()})
    y = torch.empty_like(steps_in[0]["x"])
    stream = torch.cuda.current_stream(dev)

    def one_pass(events=None):
        for t, st in enumerate(steps_in):
            if events is not None:
                events[t][0].record(stream)
            ssm.scan_fwd(st["x"], st["delta"], A, st["B"], st["C"], D, st["z"], bias, h, out=y,
                         final_state_out=h)
            if events is not None:
                events[t][1].record(stream)

    settle(lambda i: one_pass(), torch, args)
    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    passes = max(args.steps, 1)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in steps_in] for _ in range(passes)]
    t0 = time.perf_counter()
    for i in range(passes):
        one_pass(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for e in evs for a, b in e]
    per_step_s = float(np.mean(step_ms)) * 1e-3
    # The same pass captured once in a HIP graph and replayed: the launches of the
    # decode steps leave the host path (the library allocates nothing and issues no
    # memset, so the chain can be captured).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    torch.cuda.synchronize()
    for _ in range(max(args.warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(passes)]
    t0 = time.perf_counter()
    for i in range(passes):
        gev[i][0].record(stream)
        graph.replay()
        gev[i][1].record(stream)
    torch.cuda.synchronize()
    graph_ms_per_pass = (time.perf_counter() - t0) * 1e3 / passes
    # kernel time per decode step: the replayed steps run back to back with no
    # host work or event between them, so this is the kernel's own duration
    # (events around each eager step add a few microseconds to each)
    graph_step_s = float(np.mean([a.elapsed_time(b) for a, b in gev])) * 1e-3 / w.steps
    es = 2 if "bfloat16" in str(w.dtype) else 4
    bd = w.batch * w.dim
    step_bytes = (4 if w.gate else 3) * bd * es + 2 * w.batch * w.dstate * es + w.dim * w.dstate * 4 + \
        2 * w.dim * 4 + 2 * bd * w.dstate * 4
    ms_per_pass = elapsed * 1e3 / passes
    out = {
        "metric": "scan GElem/s (B*D*N per token step) + % HBM roofline per step",
        "value": round(w.elems / (ms_per_pass * 1e-3) / 1e9, 2), "unit": "GElem/s", "n_gpus": 1,
        "steps": passes, "warmup": args.warmup, "ms_per_step": round(ms_per_pass, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": io_dtype(w), "state_dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                   "io_dtype": str(w.dtype).replace("torch.", ""), "gate": w.gate, "decode_steps": w.steps,
                   "plan": {"variant": "decode", "in_place": True}},
        "per_step_kernel_us": round(graph_step_s * 1e6, 2),
        "per_step_eager_event_us": round(per_step_s * 1e6, 2),
        "wall_us_per_decode_step": round(ms_per_pass * 1e3 / w.steps, 2),
        "graph": {"ms_per_pass": round(graph_ms_per_pass, 5),
                  "wall_us_per_decode_step": round(graph_ms_per_pass * 1e3 / w.steps, 2),
                  "value": round(w.elems / (graph_ms_per_pass * 1e-3) / 1e9, 2),
                  "note": "one pass of the decode steps captured in a HIP graph and replayed"},
        "roofline": _roofline(step_bytes, graph_step_s, "scan_decode_kernel"),
    }
    out["roofline"]["traffic"] = stored_traffic(w.name)
    if not args.no_cpu_baseline:
        import torch as _t
        cpu = {k: [] for k in ("x", "delta", "B", "C", "z")}
        for t in range(w.steps):
            st = workloads.make_decode_step(w, t)
            for k in cpu:
                if st[k] is not None:
                    cpu[k].append(st[k])
        stacked = {k: (_t.cat(v, dim=1) if v else None) for k, v in cpu.items()}
        stacked.update({k: inp[k] for k in ("A", "D", "delta_bias", "h0")})
        log("cpu baseline (oracle over the stacked decode steps) ...")
        out["cpu_baseline"] = cpu_baseline(
            w, stacked, what=f"the {w.steps} decode steps as one L={w.steps} oracle scan from the workload's h0 "
                             f"(equal to {w.steps} single-token steps)")
    return out


def time_calls(fn, torch, dev, args):
    """Mean seconds per call of fn on torch's current stream (HIP events), after warmup."""
    stream = torch.cuda.current_stream(dev)
    settle(lambda i: fn(), torch, args)
    for _ in range(max(args.warmup, 1)):
        fn()
    torch.cuda.synchronize()
    n = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3


def bench_backward(w, args, ssm, torch):
    """One step = one ssm_scan_bwd over the workload: every gradient (x, delta,
    z, A, B, C, D, delta_bias, h0) from dy (and dhT when the workload returns
    the final state), states recomputed from the inputs inside the call."""
    import workloads
    dev = torch.device("cuda:0")
    log(f"workload {w.describe()} (backward)")
    inp = workloads.make_inputs(w)
    cot = workloads.make_cotangents(w)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    dy = cot["dy"].to(dev)
    dhT = cot["dhT"].to(dev) if w.final_state else None
    names = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")
    grads = {k: torch.empty_like(d[k]) for k in names if k != "h0" and d[k] is not None}
    grads["h0"] = torch.empty(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev)
    ck, fwd_ck = None, None
    if args.checkpoints:
        # the training forward: y plus the states the backward starts its chunks from
        ck = torch.empty(ssm.checkpoint_shape(w.batch, w.seqlen, w.dim, w.dstate), dtype=torch.float32, device=dev)
        y = torch.empty_like(d["x"])
        fwd_ck = time_calls(lambda: ssm.scan_fwd(*(d[k] for k in names), out=y, checkpoints=ck,
                                                 generic_a=args.generic_a, zoh=args.zoh), torch, dev, args)
        fwd_plain = time_calls(lambda: ssm.scan_fwd(*(d[k] for k in names), out=y, generic_a=args.generic_a,
                                                    zoh=args.zoh), torch, dev, args)
        ssm.scan_fwd(*(d[k] for k in names), out=y, checkpoints=ck, generic_a=args.generic_a, zoh=args.zoh)
        torch.cuda.synchronize()
        log(f"forward with checkpoints {fwd_ck * 1e3:.3f} ms, without {fwd_plain * 1e3:.3f} ms")
    a0 = ssm.make_bwd_args(*(d[k] for k in names), dy=dy, dhT=dhT, grads=grads, time_splits=args.time_splits,
                           generic_a=args.generic_a, zoh=args.zoh, checkpoints=ck)
    nbytes = ssm.bwd_workspace_bytes(a0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    a0.workspace, a0.workspace_bytes = ws.data_ptr(), nbytes
    splits = ssm.bwd_plan(a0)
    log(f"time segments {splits}, workspace {nbytes} B")
    lib = ssm.lib()
    import ctypes
    stream = torch.cuda.current_stream(dev)

    def step():
        rc = lib.ssm_scan_bwd(ctypes.byref(a0), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"ssm_scan_bwd: {ssm.strerror(rc)}")

    settle(lambda i: step(), torch, args)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    es = 2 if "bfloat16" in str(w.dtype) else 4
    bld, bln, bdn = w.batch * w.seqlen * w.dim, w.batch * w.seqlen * w.dstate, w.batch * w.dim * w.dstate
    n_tok = 4 if w.gate else 3  # (B, L, D) tensors read: x, delta, dy, (z)
    alg = (n_tok + n_tok - 1) * bld * es  # and written: dx, ddelta, (dz)
    alg += 4 * bln * es  # B, C read; dB, dC written
    alg += 2 * w.dim * w.dstate * 4 + 4 * w.dim * 4  # A read, dA written; D, bias read, dD, dbias written
    alg += bdn * 4 * (2 if w.final_state else 1) + (bdn * 4 if w.h0_std > 0 else 0)  # dhT, dh0, h0
    if ck is not None:
        alg += ck.numel() * 4  # the checkpoints read back
    ms_per_step = elapsed * 1e3 / steps
    out = {
        "metric": "backward scan GElem/s (B*L*D*N) + % HBM roofline",
        "value": round(w.elems / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GElem/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": io_dtype(w), "state_dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "dstate": w.dstate, "io_dtype": str(w.dtype).replace("torch.", ""), "gate": w.gate,
                   "time_splits": splits, "workspace_bytes": nbytes,
                   "input_term": "zero-order hold" if args.zoh else "Euler",
                   "states": "from the forward's checkpoints" if ck is not None else "recomputed"},
        "roofline": dict(_roofline(alg, call_s, "ssm_scan_bwd (local, combine, main, two reductions)"),
                         traffic=stored_traffic(w.name + ("_bwd_zoh" if args.zoh else "_bwd")
                                                + ("_checkpoints" if ck is not None else ""), BACKWARD_SOURCES)),
    }
    if ck is not None:
        out["forward_with_checkpoints_ms"] = round(fwd_ck * 1e3, 4)
        out["forward_without_checkpoints_ms"] = round(fwd_plain * 1e3, 4)
        out["checkpoint_bytes"] = ck.numel() * 4
    if not args.no_cpu_baseline:
        import oracle
        nd = min(w.dim, 512)
        sub = {k: v for k, v in inp.items()}
        for k in ("x", "delta", "z"):
            if sub[k] is not None:
                sub[k] = sub[k][:1, :, :nd]
        for k in ("B", "C"):
            sub[k] = sub[k][:1]
        sub["A"] = sub["A"][:nd]
        for k in ("D", "delta_bias"):
            sub[k] = sub[k][:nd]
        if sub["h0"] is not None:
            sub["h0"] = sub["h0"][:1, :nd]
        dys = cot["dy"][:1, :, :nd]
        dhs = cot["dhT"][:1, :nd] if w.final_state else None
        log(f"cpu baseline (oracle backward, batch row 0, {nd} channels) ...")
        t = time.perf_counter()
        oracle.scan_bwd(*(sub[k] for k in names), dy=dys, dhT=dhs, zoh=args.zoh)
        sec = time.perf_counter() - t
        el = w.seqlen * nd * w.dstate
        out["cpu_baseline"] = {
            "value": round(el / sec / 1e9, 5), "unit": "GElem/s", "cores": 1, "kind": "oracle",
            "sample": f"batch row 0, channels 0..{nd - 1}, all {w.seqlen} tokens ({el} elements), fp64 "
                      f"reverse-mode oracle, single thread; {sec:.2f} s including input widening",
        }
    return out


def bench_conv(w, args, ssm, torch):
    """One step = one ssm_conv1d_silu_fwd (width 4, bias, zero padding) over the
    workload's x: u = SiLU(causal depthwise conv(x)), the block's prologue."""
    import workloads
    dev = torch.device("cuda:0")
    log(f"workload {w.describe()} (conv1d + SiLU prologue)")
    x = workloads.make_inputs(w)["x"]
    prm = workloads.make_conv_params(w)
    xs = [x.to(dev), x.to(dev)]  # alternate so the previous step's rows are not in the LLC
    wt, bs = prm["weight"].to(dev), prm["bias"].to(dev)
    us = [torch.empty_like(xs[0]) for _ in xs]
    stream = torch.cuda.current_stream(dev)
    settle(lambda i: ssm.conv1d_silu(xs[i % 2], wt, bs, out=us[i % 2]), torch, args)
    for i in range(args.warmup):
        ssm.conv1d_silu(xs[i % 2], wt, bs, out=us[i % 2])
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        ssm.conv1d_silu(xs[i % 2], wt, bs, out=us[i % 2])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    es = 2 if "bfloat16" in str(w.dtype) else 4
    bld = w.batch * w.seqlen * w.dim
    alg = 2 * bld * es + w.dim * 4 * 4 + w.dim * 4  # x read, u written, taps and bias
    ms = elapsed * 1e3 / steps
    out = {
        "metric": "conv1d+SiLU prologue GElem/s (B*L*D) + % HBM roofline",
        "value": round(bld / (ms * 1e-3) / 1e9, 2), "unit": "GElem/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": io_dtype(w), "data": "synthetic",
        "config": {"workload": w.name, "pass": "conv1d_silu", "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "width": 4, "io_dtype": str(w.dtype).replace("torch.", "")},
        "roofline": _roofline(alg, kern_s, "conv_silu_kernel"),
    }
    if not args.no_cpu_baseline:
        import oracle
        nd = min(w.dim, 256)
        t = time.perf_counter()
        oracle.conv1d_silu(x[:, :, :nd], prm["weight"][:nd], prm["bias"][:nd])
        sec = time.perf_counter() - t
        el = w.batch * w.seqlen * nd
        out["cpu_baseline"] = {"value": round(el / sec / 1e9, 5), "unit": "GElem/s", "cores": 1, "kind": "oracle",
                               "sample": f"channels 0..{nd - 1} of every batch row and token ({el} elements), fp64 "
                                         f"oracle, single thread; {sec:.2f} s including input widening"}
    return out


def bench_ssd(args, ssm, torch):
    """One step = one ssm_ssd_fwd over a Mamba-2-shaped layer (default B4 L8192
    H64 P64 G1 N128, bf16, hT returned).  With few (b, h) pairs the library cuts
    time into segments: a step is then both launches (state-only pass, full pass)."""
    import workloads
    w = workloads.SSD_BY_NAME[args.ssd]
    dev = torch.device("cuda:0")
    log(f"workload {w.describe()}")
    inp = workloads.make_ssd_inputs(w)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    xs = [d["x"], d["x"].clone()]  # alternate so the previous step's x is not in the LLC
    names = ("dt", "A", "B", "C", "D", "dt_bias")
    ys = [torch.empty_like(xs[0]) for _ in xs]
    hT = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # segment summaries (time-split calls): allocated here, outside the timed region
    a0 = ssm.make_ssd_args(xs[0], *(d[k] for k in names), None, hT, ys[0], time_splits=args.time_splits)
    nws = ssm.ssd_workspace_bytes(a0)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    a0.workspace, a0.workspace_bytes = (ws.data_ptr() if nws else None), nws
    splits = ssm.ssd_plan(a0)
    log(f"time segments {splits}, workspace {nws} B")

    def step(i):
        ssm.ssd_fwd(xs[i % 2], *(d[k] for k in names), None, out=ys[i % 2], final_state_out=hT,
                    time_splits=args.time_splits, workspace=ws)

    settle(step, torch, args)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    toks = w.batch * w.seqlen * w.nheads
    alg = (2 * toks * w.headdim * 2 + toks * 2 + 2 * w.batch * w.seqlen * w.ngroups * w.dstate * 2
           + w.batch * w.nheads * w.headdim * w.dstate * 4 + 3 * w.nheads * 4)  # x, y, dt, B, C, hT, A/D/bias
    Q, N, P = 64, w.dstate, w.headdim
    # the method's own work: per token and head, the state update (N P multiply-adds) and the readout
    # (N P multiply-adds), 4 N P flops; the chunked form does 2 (Q N + Q P + 2 N P) on the matrix cores
    method_flops = toks * 4 * N * P
    chunked_flops = toks * 2 * (Q * N + Q * P + 2 * N * P)
    ms = elapsed * 1e3 / steps
    roof = _roofline(alg, kern_s, "ssd_fwd_kernel" if splits == 1 else "ssd_fwd_kernel, state-only + full pass")
    roof["traffic"] = stored_traffic(w.name, SSD_SOURCES)
    roof["method_tflops"] = round(method_flops / kern_s / 1e12, 2)
    roof["method_frac_bf16_dense"] = round(method_flops / kern_s / 2.5e15, 4)
    roof["chunked_form_tflops"] = round(chunked_flops / kern_s / 1e12, 2)
    out = {
        "metric": "SSD layer GElem/s (B*L*H*P*N) + % HBM roofline",
        "value": round(w.elems / (ms * 1e-3) / 1e9, 2), "unit": "GElem/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "ngroups": w.ngroups, "dstate": w.dstate, "chunk": Q,
                   "time_splits": splits},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import oracle
        t = time.perf_counter()
        oracle.ssd(inp["x"][:1], inp["dt"][:1], inp["A"], inp["B"][:1], inp["C"][:1], D=inp["D"],
                   dt_bias=inp["dt_bias"])
        sec = time.perf_counter() - t
        el = w.seqlen * w.nheads * w.headdim * w.dstate
        out["cpu_baseline"] = {"value": round(el / sec / 1e9, 5), "unit": "GElem/s", "cores": 1, "kind": "oracle",
                               "sample": f"batch row 0, all {w.nheads} heads and {w.seqlen} tokens ({el} state "
                                         f"updates), fp64 recurrence, single thread; {sec:.2f} s including input widening"}
    return out


def bench_gla(args, ssm, torch):
    """One step = one ssm_gla_fwd over a gated-linear-attention / mLSTM layer
    (default B4 L8192 H64 P64 G1 N128 with forget and input gates, bf16, hT
    returned)."""
    import workloads
    w = workloads.GLA_BY_NAME[args.gla]
    dev = torch.device("cuda:0")
    log(f"workload {w.describe()}")
    inp = workloads.make_gla_inputs(w)
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    vs = [d["v"], d["v"].clone()]  # alternate so the previous step's v is not in the LLC
    ys = [torch.empty_like(vs[0]) for _ in vs]
    hT = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # the feature map's once-per-call pass needs a workspace; allocated here, outside the timed region
    # (and the time-segment summaries)
    a0 = ssm.make_gla_args(d["q"], d["k"], vs[0], d["log_f"], d["in_gate"], None, hT, ys[0], w.feature_map,
                           args.time_splits)
    nws = ssm.gla_workspace_bytes(a0)
    ws = torch.empty(max(nws, 0), dtype=torch.uint8, device=dev)
    a0.workspace, a0.workspace_bytes = (ws.data_ptr() if nws else None), nws
    splits = ssm.gla_plan(a0)
    log(f"time segments {splits}, workspace {nws} B")

    def step(i):
        ssm.gla_fwd(d["q"], d["k"], vs[i % 2], d["log_f"], d["in_gate"], None, feature_map=w.feature_map,
                    out=ys[i % 2], final_state_out=hT, workspace=ws, time_splits=args.time_splits)

    settle(step, torch, args)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    toks = w.batch * w.seqlen * w.nheads
    alg = (2 * toks * w.headdim * 2 + 2 * w.batch * w.seqlen * w.ngroups * w.dstate * 2
           + (2 * toks * 4 if w.gated else 0) + w.batch * w.nheads * w.headdim * w.dstate * 4)  # v, y, q, k, gates, hT
    Q, N, P = 64, w.dstate, w.headdim
    # the recurrence's own work per token and head: state update and readout, 4 N P flops; the chunked form
    # does 2 (Q N + Q P + 2 N P) on the matrix cores (Q K^T, M V, Q S^T, the state update)
    method_flops = toks * 4 * N * P
    chunked_flops = toks * 2 * (Q * N + Q * P + 2 * N * P)
    ms = elapsed * 1e3 / steps
    roof = _roofline(alg, kern_s, "ssd_fwd_kernel" if splits == 1 else "ssd_fwd_kernel, state-only + full pass")
    roof["traffic"] = stored_traffic(w.name, SSD_SOURCES)
    roof["method_tflops"] = round(method_flops / kern_s / 1e12, 2)
    roof["method_frac_bf16_dense"] = round(method_flops / kern_s / 2.5e15, 4)
    roof["chunked_form_tflops"] = round(chunked_flops / kern_s / 1e12, 2)
    out = {
        "metric": "gated linear attention GElem/s (B*L*H*P*N) + % HBM roofline",
        "value": round(w.elems / (ms * 1e-3) / 1e9, 2), "unit": "GElem/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "ngroups": w.ngroups, "dstate": w.dstate, "gated": w.gated,
                   "feature_map": "elu+1" if w.feature_map else None, "chunk": Q, "time_splits": splits,
                   **({"feature_map_pass": "once per call, into the workspace"} if w.feature_map else {})},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import oracle
        t = time.perf_counter()
        one = lambda k: None if inp[k] is None else inp[k][:1]
        oracle.gla(inp["q"][:1], inp["k"][:1], inp["v"][:1], log_f=one("log_f"), in_gate=one("in_gate"),
                   feature_map=w.feature_map)
        sec = time.perf_counter() - t
        el = w.seqlen * w.nheads * w.headdim * w.dstate
        out["cpu_baseline"] = {"value": round(el / sec / 1e9, 5), "unit": "GElem/s", "cores": 1, "kind": "oracle",
                               "sample": f"batch row 0, all {w.nheads} heads and {w.seqlen} tokens ({el} state "
                                         f"updates), fp64 recurrence, single thread; {sec:.2f} s including input widening"}
    return out


def main():
    import workloads
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=workloads.WORKLOADS[2].name, choices=list(workloads.BY_NAME))
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--time-splits", type=int, default=0)
    ap.add_argument("--generic-a", action="store_true", help="never take the structured-decay path")
    ap.add_argument("--zoh", action="store_true", help="zero-order-hold input term instead of the Euler one")
    ap.add_argument("--carry-scan", action="store_true",
                    help="time-split calls compose segment summaries with the wave-level scan launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed calls of the step for this long before the warmup steps (clock ramp; 0: none)")
    ap.add_argument("--backward", action="store_true", help="time ssm_scan_bwd (all gradients) instead")
    ap.add_argument("--checkpoints", action="store_true",
                    help="with --backward: the backward starts from the forward's checkpoints (the forward writing "
                         "them is timed on its own and reported beside)")
    ap.add_argument("--prologue", action="store_true", help="time the conv1d + SiLU prologue on x instead")
    ap.add_argument("--ssd", nargs="?", const="mamba2_B4_L8192_H64_P64_N128", default=None, metavar="WORKLOAD",
                    help="time the Mamba-2 SSD layer instead")
    ap.add_argument("--gla", nargs="?", const="mlstm_B4_L8192_H64_P64_N128", default=None, metavar="WORKLOAD",
                    help="time the gated-linear-attention / mLSTM layer instead")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the scan, copy a MIB-MiB buffer `steps` times (calibrates the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the scan shards by batch or "
              "channel with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import mamba_selective_scan_06_amd as ssm

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t) / max(args.steps, 1)
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                          "seconds_per_copy": dt, "GBps": 2 * n * 4 / dt / 1e9}), flush=True)
        return

    if args.ssd:
        emit(bench_ssd(args, ssm, torch))
        return
    if args.gla:
        emit(bench_gla(args, ssm, torch))
        return
    w = workloads.BY_NAME[args.workload]
    if args.prologue:
        if w.chunks > 1 or w.steps:
            print("--prologue runs the single-call workloads", file=sys.stderr)
            sys.exit(2)
        emit(bench_conv(w, args, ssm, torch))
        return
    if args.backward:
        if w.chunks > 1 or w.steps:
            print("--backward runs the single-call workloads", file=sys.stderr)
            sys.exit(2)
        emit(bench_backward(w, args, ssm, torch))
        return
    if w.chunks > 1:
        emit(bench_chunked(w, args, ssm, torch))
        return
    if w.steps:
        emit(bench_decode(w, args, ssm, torch))
        return
    dev = torch.device("cuda:0")
    log(f"workload {w.describe()}")
    t0 = time.time()
    inp = workloads.make_inputs(w)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    d1 = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    # a second copy of the token tensors: alternating between the two keeps the
    # previous step's inputs out of the 256 MB last-level cache
    d2 = dict(d1)
    for k in ("x", "delta", "z", "B", "C"):
        if d1[k] is not None:
            d2[k] = d1[k].clone()
    sets = [d1, d2]
    y = [torch.empty_like(d1["x"]) for _ in sets]
    hT = [torch.empty(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev) for _ in sets]
    a0 = ssm.make_args(d1["x"], d1["delta"], d1["A"], d1["B"], d1["C"], d1["D"], d1["z"], d1["delta_bias"],
                       d1["h0"], hT[0], y[0], None, args.variant, args.time_splits, args.generic_a, args.zoh)
    nbytes = ssm.workspace_bytes(a0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    a0.workspace = None if ws is None else ws.data_ptr()
    a0.workspace_bytes = nbytes
    plan = ssm.plan(a0)
    log(f"plan {plan}, workspace {nbytes} B")

    def step(i):
        s = sets[i % 2]
        ssm.scan_fwd(s["x"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["delta_bias"], s["h0"],
                     out=y[i % 2], final_state_out=hT[i % 2], workspace=ws, variant=args.variant,
                     time_splits=args.time_splits, generic_a=args.generic_a, zoh=args.zoh, carry_scan=args.carry_scan)

    settle(step, torch, args)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    log(f"timed {args.steps} steps in {elapsed * 1e3:.2f} ms; per-launch ms median {np.median(kern_ms):.4f}")

    ms_per_step = elapsed * 1e3 / args.steps
    elems = w.elems
    value = elems / (ms_per_step * 1e-3) / 1e9
    kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    alg = algorithmic_bytes(w)
    achieved = alg / kern_avg_s / 1e9
    traffic = stored_traffic(w.name + ("_zoh" if args.zoh else ""))  # counters of the kernel this line runs
    out = {
        "metric": "scan GElem/s (B*L*D*N) + % HBM roofline, B4 L8192 D4096 N16 bf16",
        "value": round(value, 2),
        "unit": "GElem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": io_dtype(w),
        "state_dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim, "dstate": w.dstate,
            "io_dtype": str(w.dtype).replace("torch.", ""), "gate": w.gate, "final_state": w.final_state,
            "plan": {"variant": plan[0], "time_splits": plan[1], "generic_a": args.generic_a},
            "discretisation": "zoh" if args.zoh else "euler",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "scan_nsplit_kernel" if plan[0] == "nsplit" else f"scan_{plan[0]}_kernel",
            "kernel_avg_us": round(kern_avg_s * 1e6, 2),
            "algorithmic_bytes": alg,
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w, inp, zoh=args.zoh)
        log(f"cpu baseline {out['cpu_baseline']['value']} GElem/s on {out['cpu_baseline']['cores']} threads")
    emit(out)


if __name__ == "__main__":
    main()
