"""Benchmark of the diagonal affine scan, forward + backward, on one MI355X.

A step is one forward scan (out and the fp32 final state) followed by one
reverse-time backward (grad_a, grad_b) over one batch of synthetic inputs,
both through the C ABI with the library's automatic algorithm choice.  The
inputs are generated (seeded) and copied to HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

With no --workload, one JSON line per large workload is printed: wide
(B8 T2048 D2560 bf16), long32 (B4 T8192 D4096 fp32), longseq (B1 T131072
D1024 bf16) and, last, masked (B16 T4096 D2560 bf16, padding and reset
steps), the largest by elements.  Each line's `value` is the effective HBM
bandwidth of the whole step: the algorithmic bytes (forward 3*s*N + 4*B*D,
backward 5*s*N, s the I/O element size, N = B*T*D) divided by the mean step
time over K steps, each timed with HIP events with the Infinity Cache flushed
before it (a 1 GiB read outside the events).  Beside it: the same steps back
to back ("warm"), the forward and backward kernels' mean durations inside the
timed steps (the dominant one's roofline), the achievable ceiling of plain
streaming kernels with the step's access pattern on the same arrays, timed
the same way, and the fp64 oracle's rate on a bounded sample on the host.

    python bench.py --sweep lanes|short|tiles|complex|samu [--steps K]

prints instead the measurements behind the automatic algorithm and tile
choice, one JSON line per shape (see sweep_lines).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
# every kernel computes in fp32 (state, maps, gradients); bf16 is only the storage type
ARITH_DTYPE = "f32"

WORKLOAD_TEXT = {
    "small": "B=2 T=256 D=64 fp32, a~U(0.9,0.999), b=N(0,1)*sqrt(1-a^2)",
    "wide": "B=8 T=2048 D=2560 bf16 I/O fp32 state, a=clip(sigmoid(N(4,1)),0.8,0.9999), b=N(0,1)*sqrt(1-a^2)",
    "long32": "B=4 T=8192 D=4096 fp32, a~U(0.95,0.9999), b~N(0,1)",
    "longseq": "B=1 T=131072 D=1024 bf16 I/O fp32 state, a~U(0.99,0.99999), b~N(0,0.1)",
    "masked": "B=16 T=4096 D=2560 bf16, a~U(0.5,0.9999), 10% padding / 5% reset tokens",
    "cwide": "complex, planar re/im: B=8 T=2048 M=2560 bf16 I/O fp32 state, a=r*exp(i*theta), "
             "r=clip(sigmoid(N(4,1)),0.8,0.9999), theta~U(-pi/8,pi/8), b=CN(0,1)*sqrt((1-r^2)/2)",
    "csmall": "complex, planar re/im: B=2 T=256 M=64 fp32, the cwide recipe",
    "swide": "fused transition (SAMU form), planar re/im: B=8 T=2048 M=2560 bf16 I/O fp32 state, "
             "a=exp(-e^nu_log e^eta) exp(i(e^theta_log+delta)) rebuilt in the kernel, "
             "nu~U(0.005,0.5), theta~U(0.001,pi), eta~N(0,0.5^2), delta~N(0,0.1^2), b=0.3 CN(0,1)",
    "ssmall": "fused transition (SAMU form): B=2 T=256 M=64 fp32, the swide recipe",
}


def algorithmic_bytes(B, T, D, s):
    N = B * T * D
    return 3 * s * N + 4 * B * D, 5 * s * N


# The sources each family of tiled kernels is built from: counter readings are
# only valid for the sources they were taken on.
KERNEL_SOURCES = {
    "real": ("fused.hip", "fused_common.hpp", "device.hpp"),
    "complex": ("complex.hip", "complex_math.hpp", "fused_common.hpp", "device.hpp"),
    "samu": ("samu.hip", "complex_math.hpp", "fused_common.hpp", "device.hpp"),
}


def code_only(text):
    """C++ source with its comments removed and its whitespace collapsed, so
    that a change to a comment is not a change to the kernel (the sources
    hold no string literal with a comment marker in it)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sources_sha256(family="real", read=None):
    """Hash of one kernel family's sources, comments and layout left out.
    `read(name)` returns a source file's text (default: the working tree)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_recurrence_sequence_diag_amd", "csrc")
    for f in KERNEL_SOURCES[family]:
        if read is None:
            with open(os.path.join(csrc, f)) as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(code_only(text).encode())
    return h.hexdigest()


def measured_traffic(workload, direction, algo, family="real"):
    """HBM bytes per launch of the dominant kernel from the rocprofv3 counter
    runs recorded in profiles/hbm_traffic.json (FETCH_SIZE and WRITE_SIZE in
    KiB per dispatch, each scaled by what the counter reads for a plain copy of
    known size).  None when no reading exists for this kernel or its sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if algo != "fused" or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    w = rec.get("workloads", {}).get(workload, {})
    if w.get("source_sha256", rec.get("source_sha256")) != kernel_sources_sha256(family):
        return None
    e = w.get(direction)
    if not e:
        return None
    cf = rec["copy_factor"]
    kib = e["fetch_kib"] * cf["FETCH_SIZE"] + e["write_kib"] * cf["WRITE_SIZE"]
    return round(kib * 1024)


def back_to_back_ms(torch, stream, fns, steps):
    """Mean time (ms) of `steps` back-to-back runs of fns, by HIP events."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        for f in fns:
            f()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def roofline(kernel, nbytes, ms, traffic=None):
    """The dominant kernel's HBM roofline entry: algorithmic bytes per launch
    over its average launch interval, against MI355X's 8 TB/s."""
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}


def timed_sample(fn, budget_s):
    """Run fn() repeatedly for about budget_s; returns (passes, seconds)."""
    reps, t_total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        fn()
        t_total += time.perf_counter() - t0
        reps += 1
        if t_total >= budget_s or reps >= 200:
            return reps, t_total


def cpu_baseline(inp, budget_s=10.0):
    """The fp64 oracle on the host cores, on a bounded sample of the same
    workload: batch row 0 (every step and lane of it), fwd+bwd, repeated for
    about `budget_s`; one pass on a single thread over the first lanes of row
    0 beside it.  Returns a dict."""
    import oracle

    import workloads as W

    wl = inp.workload
    cores = min(16, len(os.sched_getaffinity(0)))
    a, b, g = (W.storage_to_f64(getattr(inp, n)[:1], wl.dtype) for n in ("a", "b", "g"))

    def run(x, y, z, threads):
        h, _ = oracle.scan_fwd(x, y, threads=threads)
        oracle.scan_bwd(x, h, z, threads=threads)
    reps, t_total = timed_sample(lambda: run(a, b, g, cores), budget_s)
    # one pass on a single core over the first lanes of row 0
    d1 = min(wl.D, 256)
    a1, b1, g1 = (np.ascontiguousarray(x[:, :, :d1]) for x in (a, b, g))
    t0 = time.perf_counter()
    run(a1, b1, g1, 1)
    t_one = time.perf_counter() - t0
    fb, bb = algorithmic_bytes(1, wl.T, wl.D, wl.itemsize)
    f1, b1b = algorithmic_bytes(1, wl.T, d1, wl.itemsize)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round((fb + bb) * reps / t_total / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"batch row 0 of the {wl.name} workload ([1, {wl.T}, {wl.D}]), fwd+bwd, "
                  f"{reps} pass(es) in {t_total:.1f} s (fp64, {cores} threads over lanes; "
                  f"input conversion untimed)",
        "elements_per_s": round(wl.T * wl.D * reps / t_total, 1),
        "single_core": {"value": round((f1 + b1b) / t_one / 1e9, 3), "unit": "GB/s",
                        "sample": f"lanes 0..{d1 - 1} of batch row 0, one fwd+bwd pass in "
                                  f"{t_one:.2f} s on 1 thread"},
        "host": {"cpu_model": model, "hardware_threads": os.cpu_count()},
    }


def complex_line(args, wl, lr, torch, W):
    """JSON line of the complex scan (planar re/im arrays): train = forward +
    backward through AUTO; prefill = the state-only forward."""
    inp = W.generate_complex(wl, seed=0)
    B, T, M = wl.B, wl.T, wl.D
    s = wl.itemsize
    N = B * T * M

    def dev(x):
        if wl.dtype == "f32":
            return torch.from_numpy(x).cuda()
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)

    ar, ai, br, bi, gr, gi = (dev(getattr(inp, n)) for n in ("ar", "ai", "br", "bi", "gr", "gi"))
    dt = lr.F32 if wl.dtype == "f32" else lr.BF16
    out_r, out_i = torch.empty_like(ar), torch.empty_like(ar)
    g4 = [torch.empty_like(ar) for _ in range(4)]
    last = [torch.empty((B, M), device="cuda", dtype=torch.float32) for _ in range(2)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    o = lr.make_opts(algo=args.algo)
    P = lambda t: t.data_ptr()

    def fwd(with_out=True):
        lr.scan_complex_fwd(P(ar), P(ai), P(br), P(bi), P(out_r) if with_out else None,
                            P(out_i) if with_out else None, P(last[0]), P(last[1]), None, None,
                            B, T, M, dt, sh, o)

    def bwd():
        lr.scan_complex_bwd(P(ar), P(ai), P(out_r), P(out_i), P(gr), P(gi), None, None, None,
                            None, P(g4[0]), P(g4[1]), P(g4[2]), P(g4[3]), None, None, B, T, M, dt,
                            sh, o)

    if args.mode == "prefill":
        step = [lambda: fwd(False)]
        nbytes = 4 * s * N + 8 * B * M
    else:
        step = [fwd, bwd]
        nbytes = (6 * s * N + 8 * B * M) + 10 * s * N
    for _ in range(args.warmup):
        for f in step:
            f()
    torch.cuda.synchronize()
    if args.mode == "prefill":
        ms = back_to_back_ms(torch, stream, step, args.steps)
    else:
        (fwd_ms, bwd_ms), ms, warm_ms = step_times(torch, stream, step, args.steps,
                                                    cache_flush(torch))
    res = {"metric": f"complex {args.mode}: effective HBM GB/s",
           "value": round(nbytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": ARITH_DTYPE,
           "data": "synthetic (seeded numpy draws, see workloads/__init__.py)",
           "config": {"workload": f"{wl.name}: {WORKLOAD_TEXT[wl.name]}", "B": B, "T": T, "M": M,
                      "io_dtype": wl.dtype}}
    res["pct_of_peak"] = round(100 * res["value"] / HBM_PEAK_GBPS, 2)
    if args.mode != "prefill":
        res["timing"] = COLD_TIMING
        for name, kms, nb in (("fwd", fwd_ms, 6 * s * N + 8 * B * M), ("bwd", bwd_ms, 10 * s * N)):
            res[f"{name}_us"] = round(kms * 1e3, 2)
            res[f"{name}_GBps"] = round(nb / (kms * 1e-3) / 1e9, 1)
        res["warm"] = {"ms_per_step": round(warm_ms, 5),
                       "value": round(nbytes / (warm_ms * 1e-3) / 1e9, 2),
                       "note": "K steps back to back, no flush"}
        res["roofline"] = roofline("complex backward scan (fused)", 10 * s * N, bwd_ms,
                                   measured_traffic(wl.name, "backward", "fused", "complex"))
    else:
        # no counter run covers the state-only kernel (it stores only `last`)
        res["roofline"] = roofline("complex state-only forward (fused)", nbytes, ms)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = complex_cpu_baseline(inp, args.mode)
    return res


def complex_cpu_baseline(inp, mode, budget_s=8.0):
    """The fp64 complex oracle (one host thread) on batch row 0 of the
    workload, fwd+bwd (or the forward alone for prefill), scaled to GB/s with
    the same algorithmic bytes per element."""
    import oracle

    wl = inp.workload
    lanes = [(0, m) for m in range(wl.D)]
    a, b, g = inp.c128("a", lanes), inp.c128("b", lanes), inp.c128("g", lanes)
    s, N1 = wl.itemsize, wl.T * wl.D

    def run():
        h, _ = oracle.complex_fwd(a, b)
        if mode != "prefill":
            oracle.complex_bwd(a, h, g)
    reps, t = timed_sample(run, budget_s)
    nb = (4 * s * N1 + 8 * wl.D) if mode == "prefill" else (6 * s * N1 + 8 * wl.D + 10 * s * N1)
    return {"value": round(nb * reps / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"batch row 0 of {wl.name} ([1, {wl.T}, {wl.D}]), "
                      f"{'forward' if mode == 'prefill' else 'fwd+bwd'}, {reps} pass(es) in {t:.1f} s "
                      f"(fp64 C99 complex, one thread; input conversion untimed)"}


def samu_line(args, wl, lr, torch, W):
    """JSON line of the fused-transition scan: train = forward + backward
    (all four parameter gradients and grad_b); prefill = the state-only
    forward.  Algorithmic bytes count the arrays of the interface only: the
    forward reads b (re, im), eta, delta, nu_log, theta_log and writes out
    (re, im) and last; the backward reads out, grad_out (re, im each), the
    controls and parameters and writes grad_b (re, im) and the four
    parameter gradients."""
    inp = W.generate_samu(wl, seed=0)
    B, T, M = wl.B, wl.T, wl.D
    s = wl.itemsize
    N = B * T * M

    def dev(x):
        if wl.dtype == "f32":
            return torch.from_numpy(x).cuda()
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)

    eta, delta, br, bi, gr, gi = (dev(getattr(inp, n))
                                  for n in ("eta", "delta", "br", "bi", "gr", "gi"))
    nu_log = torch.from_numpy(inp.nu_log).cuda()
    theta_log = torch.from_numpy(inp.theta_log).cuda()
    dt = lr.F32 if wl.dtype == "f32" else lr.BF16
    out_r, out_i = torch.empty_like(br), torch.empty_like(br)
    gbr, gbi = torch.empty_like(br), torch.empty_like(br)
    f32 = dict(device="cuda", dtype=torch.float32)
    last = [torch.empty((B, M), **f32) for _ in range(2)]
    ge, gd = torch.empty((B, T), **f32), torch.empty((B, T), **f32)
    gn, gt = torch.empty((M,), **f32), torch.empty((M,), **f32)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    o = lr.make_opts(algo=args.algo)
    P = lambda t: t.data_ptr()
    ctl = (P(eta), P(delta), P(nu_log), P(theta_log))

    def fwd(with_out=True):
        lr.scan_samu_fwd(*ctl, P(br), P(bi), P(out_r) if with_out else None,
                         P(out_i) if with_out else None, P(last[0]), P(last[1]), None, None,
                         B, T, M, dt, sh, o)

    def bwd():
        lr.scan_samu_bwd(*ctl, P(out_r), P(out_i), P(gr), P(gi), None, None, None, None, P(ge),
                         P(gd), P(gn), P(gt), P(gbr), P(gbi), None, None, B, T, M, dt, sh, o)

    ctl_bytes = 2 * s * B * T + 8 * M
    fwd_bytes = 4 * s * N + 8 * B * M + ctl_bytes
    bwd_bytes = 6 * s * N + ctl_bytes + 8 * B * T + 8 * M
    if args.mode == "prefill":
        step = [lambda: fwd(False)]
        nbytes = 2 * s * N + 8 * B * M + ctl_bytes
    else:
        step = [fwd, bwd]
        nbytes = fwd_bytes + bwd_bytes
    for _ in range(args.warmup):
        for f in step:
            f()
    torch.cuda.synchronize()
    if args.mode == "prefill":
        ms = back_to_back_ms(torch, stream, step, args.steps)
    else:
        (fwd_ms, bwd_ms), ms, warm_ms = step_times(torch, stream, step, args.steps,
                                                    cache_flush(torch))
    res = {"metric": f"fused-transition {args.mode}: effective HBM GB/s",
           "value": round(nbytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": ARITH_DTYPE,
           "data": "synthetic (seeded numpy draws, see workloads/__init__.py)",
           "config": {"workload": f"{wl.name}: {WORKLOAD_TEXT[wl.name]}", "B": B, "T": T, "M": M,
                      "io_dtype": wl.dtype}}
    res["pct_of_peak"] = round(100 * res["value"] / HBM_PEAK_GBPS, 2)
    if args.mode != "prefill":
        res["timing"] = COLD_TIMING
        for name, kms, nb in (("fwd", fwd_ms, fwd_bytes), ("bwd", bwd_ms, bwd_bytes)):
            res[f"{name}_us"] = round(kms * 1e3, 2)
            res[f"{name}_GBps"] = round(nb / (kms * 1e-3) / 1e9, 1)
        res["warm"] = {"ms_per_step": round(warm_ms, 5),
                       "value": round(nbytes / (warm_ms * 1e-3) / 1e9, 2),
                       "note": "K steps back to back, no flush"}
        # the backward call is three launches (factor tables, the tiled
        # kernel, the fixed-order reduction); its interval is charged whole
        res["roofline"] = roofline("fused-transition backward call (fused)", bwd_bytes, bwd_ms,
                                   measured_traffic(wl.name, "backward", "fused", "samu"))
    else:
        res["roofline"] = roofline("fused-transition state-only forward call (fused)", nbytes, ms)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = samu_cpu_baseline(inp, args.mode)
    return res


def samu_cpu_baseline(inp, mode, budget_s=8.0):
    """The fp64 fused-transition oracle (one host thread) on batch row 0,
    fwd+bwd (or the forward alone for prefill), in the same GB/s."""
    import oracle

    wl = inp.workload
    rows = [0]
    eta, delta, nu_log, theta_log = inp.controls(rows)
    b, g = inp.c128("b", rows), inp.c128("g", rows)
    s, N1, T, M = wl.itemsize, wl.T * wl.D, wl.T, wl.D

    def run():
        h, _ = oracle.samu_fwd(eta, delta, nu_log, theta_log, b)
        if mode != "prefill":
            oracle.samu_bwd(eta, delta, nu_log, theta_log, h, g)
    reps, t = timed_sample(run, budget_s)
    ctl = 2 * s * T + 8 * M
    nb = (2 * s * N1 + 8 * M + ctl) if mode == "prefill" else (
        4 * s * N1 + 8 * M + ctl + 6 * s * N1 + ctl + 8 * T + 8 * M)
    return {"value": round(nb * reps / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"batch row 0 of {wl.name} ([1, {T}, {M}]), "
                      f"{'forward' if mode == 'prefill' else 'fwd+bwd'}, {reps} pass(es) in {t:.1f} s "
                      f"(fp64 C99 complex, one thread; input conversion untimed)"}


def inference_line(args, wl, lr, torch, a, b, dt, inp=None):
    """JSON line of the state-only forward (prefill) or of the decode step."""
    B, T, D = wl.B, wl.T, wl.D
    s = wl.itemsize
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    last = torch.empty((B, D), device="cuda", dtype=torch.float32)
    if args.mode == "prefill":
        o = lr.make_opts(algo=args.algo, chunk=args.fwd_chunk, width=args.fwd_width)

        def fn():
            lr.scan_fwd_ex(a.data_ptr(), b.data_ptr(), None, last.data_ptr(), B, T, D, dt, sh, o)
        nbytes = 2 * s * B * T * D + 4 * B * D
        unit_note = "state-only forward: reads a and b, writes the fp32 last state"
    else:
        # one token: a[:, t], b[:, t] as [B, D] (a strided view is made contiguous once)
        at = a[:, T // 2].contiguous()
        bt = b[:, T // 2].contiguous()
        state = torch.zeros((B, D), device="cuda", dtype=torch.float32)
        out = torch.empty_like(at)

        def fn(on=sh):
            lr.scan_step(at.data_ptr(), bt.data_ptr(), state.data_ptr(), None, out.data_ptr(),
                         state.data_ptr(), B, D, dt, on)
        nbytes = (3 * s + 8) * B * D
        unit_note = "one decode step: reads a, b and the fp32 state, writes out and the state"
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {
        "metric": f"{args.mode}: effective HBM GB/s",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": ARITH_DTYPE,
        "data": "synthetic (seeded numpy draws, see workloads/__init__.py)",
        "config": {"workload": f"{wl.name}: {WORKLOAD_TEXT[wl.name]}", "B": B, "T": T, "D": D,
                   "io_dtype": wl.dtype,
                   "mode": unit_note},
        "us_per_call": round(ms * 1e3, 2),
        **({"graph_us_per_step": round(graph_decode_us(torch, fn, stream, args.steps), 2)}
           if args.mode == "decode" else {}),
        "pct_of_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": roofline("state-only forward (fused)" if args.mode == "prefill"
                             else "decode step (one launch; launch-latency bound at this size)",
                             nbytes, ms),
        **({"cpu_baseline": inference_cpu_baseline(inp, args.mode)}
           if inp is not None and not args.no_cpu_baseline else {}),
    }


def graph_decode_us(torch, fn, stream, steps):
    """Per-step time of `steps` decode steps captured in one HIP graph and
    replayed (the launch interval of eager back-to-back calls removed);
    fn(stream_handle) enqueues one step."""
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    fn(s.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(steps):
            fn(s.cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(5):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (5 * steps)


def inference_cpu_baseline(inp, mode, budget_s=8.0):
    """The fp64 oracle beside the inference modes: the forward over the whole
    workload (prefill), or one time step on the [B, D] lanes from a carried
    state (decode), in the same GB/s."""
    import oracle

    wl = inp.workload
    cores = min(16, len(os.sched_getaffinity(0)))
    s, B, T, D = wl.itemsize, wl.B, wl.T, wl.D
    if mode == "prefill":
        a, b = inp.f64("a"), inp.f64("b")
        reps, t = timed_sample(lambda: oracle.scan_fwd(a, b, threads=cores), budget_s)
        nb, what = 2 * s * B * T * D + 4 * B * D, f"the whole {wl.name} forward"
    else:
        a, b = inp.f64("a")[:, T // 2:T // 2 + 1], inp.f64("b")[:, T // 2:T // 2 + 1]
        state = np.zeros((B, D))
        reps, t = timed_sample(lambda: oracle.scan_fwd(a, b, h0=state, threads=cores), budget_s / 4)
        nb, what = (3 * s + 8) * B * D, f"one {wl.name} time step on [B, D] lanes"
    return {"value": round(nb * reps / t / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}, {reps} pass(es) in {t:.1f} s (fp64, {cores} threads over lanes)"}


class StreamCeiling:
    """Plain streaming kernels (libstreamceil.so, built beside liblrscan.so)
    with the scan's access patterns: read 2 / write 1 and read 3 / write 2,
    non-temporal stores, each input loaded normally or non-temporally."""

    def __init__(self):
        import ctypes

        import linear_recurrence_sequence_diag_amd as lr
        path = os.path.join(os.path.dirname(lr.LIB_PATH), "libstreamceil.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run "
                              "`python -m linear_recurrence_sequence_diag_amd.build`")
        self.lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        self.lib.stream_ceiling_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P,
                                                P, P, ctypes.c_size_t, P]
        self.lib.stream_ceiling_run.restype = ctypes.c_int

    def run(self, pattern, unroll, nt_mask, ins, outs, nbytes, stream):
        p = [t.data_ptr() for t in ins] + [None] * (3 - len(ins))
        q = [t.data_ptr() for t in outs] + [None] * (2 - len(outs))
        rc = self.lib.stream_ceiling_run(pattern, unroll, nt_mask, p[0], p[1], p[2], q[0], q[1],
                                         nbytes, stream)
        if rc != 0:
            raise RuntimeError(f"stream_ceiling_run failed ({rc})")


def cold_times(torch, stream, fns, steps, flush):
    """Each of `steps` repetitions: flush the caches (outside the events),
    then run fns in order with a HIP event before, between and after them on
    `stream`.  Returns one list of durations (ms) per fn."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
          for _ in range(steps)]
    for k in range(steps):
        flush()
        ev[k][0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[k][i + 1].record(stream)
    torch.cuda.synchronize()
    return [[ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)] for i in range(len(fns))]


def cache_flush(torch):
    """The cache flush: a 1 GiB read, four times the 256 MB Infinity Cache (a
    read leaves clean lines, so the timed step pays no write-back for it)."""
    scrub = torch.ones(1 << 28, device="cuda", dtype=torch.float32)
    scrub_sum = torch.empty((), device="cuda", dtype=torch.float32)
    return lambda: torch.sum(scrub, dim=0, out=scrub_sum)


def step_times(torch, stream, fns, steps, flush):
    """The step timed as the real-scan lines time it: the mean of each call
    over `steps` cold repetitions (caches flushed before each, HIP events
    around each call), their sum, and the mean of `steps` back-to-back steps
    (ms)."""
    per = cold_times(torch, stream, fns, steps, flush)
    means = [sum(t) / len(t) for t in per]
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(steps):
        for f in fns:
            f()
    w1.record(stream)
    torch.cuda.synchronize()
    return means, sum(means), w0.elapsed_time(w1) / steps


COLD_TIMING = ("mean over K steps, each with the Infinity Cache flushed before it "
               "(a 1 GiB read outside the events)")


DEFAULT_WORKLOADS = ("wide", "long32", "longseq", "masked")


def train_line(args, name, lr, torch, W, cpu_budget):
    """JSON line of the fwd+bwd step on one of the named real workloads."""
    wl = W.WORKLOADS[name]
    inp = W.generate(wl, seed=0)
    dt = lr.F32 if wl.dtype == "f32" else lr.BF16

    def dev(x):
        if wl.dtype == "f32":
            return torch.from_numpy(x).cuda()
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)

    a, b, g = dev(inp.a), dev(inp.b), dev(inp.g)
    B, T, D = wl.B, wl.T, wl.D
    if args.mode != "train":
        return inference_line(args, wl, lr, torch, a, b, dt, inp)
    out = torch.empty_like(a)
    ga = torch.empty_like(a)
    gb = torch.empty_like(a)
    last = torch.empty((B, D), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    fo = lr.make_opts(algo=args.algo, chunk=args.fwd_chunk, width=args.fwd_width)
    bo = lr.make_opts(algo=args.algo, chunk=args.bwd_chunk, width=args.bwd_width)

    def fwd():
        lr.scan_fwd_ex(a.data_ptr(), b.data_ptr(), out.data_ptr(), last.data_ptr(), B, T, D, dt,
                       sh, fo)

    def bwd():
        lr.scan_bwd_ex(a.data_ptr(), out.data_ptr(), g.data_ptr(), None, ga.data_ptr(),
                       gb.data_ptr(), B, T, D, dt, sh, bo)

    flush = cache_flush(torch)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    # timed region: K steps, the caches flushed before each, HIP events on the
    # launch stream before, between and after the two calls (each call is
    # one kernel launch with the automatic choice)
    fwd_t, bwd_t = cold_times(torch, stream, [fwd, bwd], args.steps, flush)
    step_t = [x + y for x, y in zip(fwd_t, bwd_t)]
    ms_per_step = sum(step_t) / len(step_t)
    fwd_ms = sum(fwd_t) / len(fwd_t)
    bwd_ms = sum(bwd_t) / len(bwd_t)

    # the same steps back to back (inputs partly left in the Infinity Cache)
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(args.steps):
        fwd()
        bwd()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps

    fb, bb = algorithmic_bytes(B, T, D, wl.itemsize)
    value = (fb + bb) / (ms_per_step * 1e-3) / 1e9

    # achievable ceiling: streaming kernels with the step's access pattern on
    # the same arrays (forward: a, b -> out; backward: a, out, grad_out ->
    # grad_a, grad_b), timed like the step; the best of three unroll depths
    # and three load policies (every input normal; the scan's policy: the
    # forward's b non-temporal, everything the backward reads non-temporal;
    # every input non-temporal)
    ceil = StreamCeiling()
    nb = a.numel() * a.element_size()
    best = None
    for u in (1, 2, 4):
        for fm, bm in ((0, 0), (2, 7), (7, 7)):
            tf, tb = cold_times(torch, stream,
                                [lambda: ceil.run(1, u, fm, [a, b], [out], nb, sh),
                                 lambda: ceil.run(2, u, bm, [a, out, g], [ga, gb], nb, sh)],
                                args.steps, flush)
            c = (sum(tf) / len(tf), sum(tb) / len(tb), u, fm, bm)
            if best is None or c[0] + c[1] < best[0] + best[1]:
                best = c
    ceil_gbps = (fb + bb) / ((best[0] + best[1]) * 1e-3) / 1e9
    del flush

    fwd_algo, fwd_chunk, fwd_width = lr.scan_auto_algo(B, T, D, dt, 0)
    bwd_algo, bwd_chunk, bwd_width = lr.scan_auto_algo(B, T, D, dt, 1)
    if args.algo != "auto":
        fwd_algo = bwd_algo = lr.ALGOS[args.algo]
        fwd_chunk, bwd_chunk = args.fwd_chunk, args.bwd_chunk
        fwd_width, bwd_width = args.fwd_width, args.bwd_width
    names = {v: k for k, v in lr.ALGOS.items()}

    def algo_name(algo, chunk, width):
        if names[algo] == "fused":
            return f"fused(width {width * 16} B, tile {chunk} rows)"
        if names[algo] == "chunked":
            return f"chunked(chunk {chunk})"
        return names[algo]
    if bwd_ms >= fwd_ms:
        dom, dom_ms, dom_bytes, dom_algo = "backward", bwd_ms, bb, names[bwd_algo]
    else:
        dom, dom_ms, dom_bytes, dom_algo = "forward", fwd_ms, fb, names[fwd_algo]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

    res = {
        "metric": "fwd+bwd scan effective HBM GB/s (and % of peak), elements/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ARITH_DTYPE,
        "data": "synthetic (seeded numpy draws, see workloads/__init__.py)",
        "config": {
            "workload": f"{wl.name}: {WORKLOAD_TEXT[wl.name]}",
            "B": B, "T": T, "D": D,
            "io_dtype": wl.dtype,
            "fwd_algo": algo_name(fwd_algo, fwd_chunk, fwd_width),
            "bwd_algo": algo_name(bwd_algo, bwd_chunk, bwd_width),
        },
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "elements_per_s": round(wl.N / (ms_per_step * 1e-3), 1),
        "timing": COLD_TIMING,
        "fwd_us": round(fwd_ms * 1e3, 2),
        "bwd_us": round(bwd_ms * 1e3, 2),
        "fwd_GBps": round(fb / (fwd_ms * 1e-3) / 1e9, 1),
        "bwd_GBps": round(bb / (bwd_ms * 1e-3) / 1e9, 1),
        "step_ms_min": round(min(step_t), 5),
        "per_call_us": {"fwd_median": round(float(np.median(fwd_t)) * 1e3, 2),
                        "fwd_min": round(min(fwd_t) * 1e3, 2),
                        "bwd_median": round(float(np.median(bwd_t)) * 1e3, 2),
                        "bwd_min": round(min(bwd_t) * 1e3, 2)},
        "warm": {"ms_per_step": round(warm_ms, 5),
                 "value": round((fb + bb) / (warm_ms * 1e-3) / 1e9, 2),
                 "note": "K steps back to back, no flush"},
        "ceiling": {"kernel": "streaming kernels with the step's access pattern on the same "
                              "arrays (read 2 / write 1, read 3 / write 2), timed like the step",
                    "GB/s": round(ceil_gbps, 1),
                    "fwd_pattern_us": round(best[0] * 1e3, 2),
                    "bwd_pattern_us": round(best[1] * 1e3, 2),
                    "unroll": best[2],
                    "load_policy": {0: "normal", 2: "b non-temporal", 7: "non-temporal"}[best[3]]
                                   + " / " + {0: "normal", 7: "non-temporal"}[best[4]],
                    "value_frac": round(value / ceil_gbps, 4)},
        "roofline": {
            "bound": "hbm",
            "kernel": f"{dom} scan ({dom_algo})",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(wl.name, dom, dom_algo),
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, cpu_budget)
    return res


# Tile shapes (row width in 16-byte vectors, rows per tile) the fused form
# is built for, per direction; the library rejects any other pair.
FUSED_FWD_SHAPES = ((8, 256), (8, 512), (16, 128), (16, 256), (32, 32), (32, 64), (32, 128))
FUSED_BWD_SHAPES = ((8, 256), (8, 128), (16, 128), (32, 64), (32, 32))

SWEEP_LANES = ((8, 2048, 2560), (32, 2048, 2560), (128, 2048, 2560), (512, 512, 2560),
               (2048, 128, 2560), (8192, 32, 2560))
SWEEP_SHORT_T = (8, 16, 32, 64, 128, 256, 512, 1024)


def sweep_lines(args, lr, torch, W):
    """The measurements behind the automatic algorithm choice, one JSON line
    per point; every time is the mean of `--steps` calls, each with the
    Infinity Cache flushed before it (HIP events around the call).

    lanes: the per-lane walk against the automatic choice as the number of
      lanes B*D grows (D = 2560, bf16 and fp32).
    short: every fused tile shape, the walk and the automatic choice on
      short sequences at constant work (B*T*D*s ~ 680 MB over the three
      forward arrays, T from 8 to 1024, D = 2560).
    tiles: every fused tile shape and the automatic choice on the four large
      workloads.
    Inputs for lanes and short are drawn on the device (a ~ U(0.5, 0.9999),
    b, g ~ N(0, 1)); tiles uses the workloads' own generators.  Rates are the
    algorithmic bytes (forward 3*s*N + 4*B*D, backward 5*s*N) per second."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    flush = cache_flush(torch)
    steps = max(1, args.steps)

    def arrays(B, T, D, tdt, gen=None):
        if gen is not None:
            return gen
        g0 = torch.Generator(device="cuda")
        g0.manual_seed(0)
        a = torch.empty(B, T, D, device="cuda").uniform_(0.5, 0.9999, generator=g0).to(tdt)
        b = torch.randn(B, T, D, device="cuda", generator=g0).to(tdt)
        g = torch.randn(B, T, D, device="cuda", generator=g0).to(tdt)
        return a, b, g

    def measure(B, T, D, dt, a, b, g, variants):
        """variants: name -> (forward opts or None, backward opts or None)."""
        out = torch.empty_like(a)
        ga = torch.empty_like(a)
        gb = torch.empty_like(a)
        last = torch.empty((B, D), device="cuda", dtype=torch.float32)
        s = a.element_size()
        N = B * T * D
        fb, bb = 3 * s * N + 4 * B * D, 5 * s * N
        auto = lr.make_opts()
        lr.scan_fwd_ex(a.data_ptr(), b.data_ptr(), out.data_ptr(), last.data_ptr(), B, T, D, dt,
                       sh, auto)
        res = {}
        for name, (fo, bo) in variants.items():
            fns = []
            if fo is not None:
                fns.append(lambda fo=fo: lr.scan_fwd_ex(a.data_ptr(), b.data_ptr(), out.data_ptr(),
                                                        last.data_ptr(), B, T, D, dt, sh, fo))
            if bo is not None:
                fns.append(lambda bo=bo: lr.scan_bwd_ex(a.data_ptr(), out.data_ptr(), g.data_ptr(),
                                                        None, ga.data_ptr(), gb.data_ptr(), B, T,
                                                        D, dt, sh, bo))
            for f in fns:  # first call: workspace and code objects
                f()
            torch.cuda.synchronize()
            per = cold_times(torch, stream, fns, steps, flush)
            ms = [sum(t) / len(t) for t in per]
            r = {}
            k = 0
            if fo is not None:
                r["fwd_us"] = round(ms[k] * 1e3, 1)
                r["fwd_gbps"] = round(fb / (ms[k] * 1e-3) / 1e9, 1)
                k += 1
            if bo is not None:
                r["bwd_us"] = round(ms[k] * 1e3, 1)
                r["bwd_gbps"] = round(bb / (ms[k] * 1e-3) / 1e9, 1)
            res[name] = r
        del out, ga, gb, last
        return res

    def best(res, key):
        ranked = sorted((v[key], k) for k, v in res.items() if key in v)
        return [k for _, k in ranked[::-1][:3]]

    def shape_variants():
        v = {"walk": (lr.make_opts(algo="seq"), lr.make_opts(algo="seq")),
             "auto": (lr.make_opts(), lr.make_opts())}
        fwd = set(FUSED_FWD_SHAPES)
        bwd = set(FUSED_BWD_SHAPES)
        for w, t in sorted(fwd | bwd):
            v[f"w{w}x{t}"] = (lr.make_opts(algo="fused", width=w, chunk=t) if (w, t) in fwd else None,
                              lr.make_opts(algo="fused", width=w, chunk=t) if (w, t) in bwd else None)
        return v

    dtypes = (("bf16", lr.BF16, torch.bfloat16), ("f32", lr.F32, torch.float32))
    if args.sweep == "lanes":
        for name, dt, tdt in dtypes:
            for B, T, D in SWEEP_LANES:
                a, b, g = arrays(B, T, D, tdt)
                res = measure(B, T, D, dt, a, b, g,
                              {"walk": (lr.make_opts(algo="seq"), lr.make_opts(algo="seq")),
                               "auto": (lr.make_opts(), lr.make_opts())})
                print(json.dumps({"sweep": "lanes", "dtype": name, "B": B, "T": T, "D": D,
                                  "lanes": B * D, "steps": steps, **res}), flush=True)
                del a, b, g
                torch.cuda.empty_cache()
    elif args.sweep == "short":
        D = 2560
        for name, dt, tdt in dtypes:
            s = 2 if name == "bf16" else 4
            for T in SWEEP_SHORT_T:
                B = max(1, int(round(3.4e8 * 2 / s / (T * D))))
                a, b, g = arrays(B, T, D, tdt)
                res = measure(B, T, D, dt, a, b, g, shape_variants())
                print(json.dumps({"sweep": "short", "dtype": name, "B": B, "T": T, "D": D,
                                  "steps": steps, "best_fwd": best(res, "fwd_gbps"),
                                  "best_bwd": best(res, "bwd_gbps"), **res}), flush=True)
                del a, b, g
                torch.cuda.empty_cache()
    else:
        for wname in DEFAULT_WORKLOADS:
            wl = W.WORKLOADS[wname]
            inp = W.generate(wl, seed=0)
            dt = lr.F32 if wl.dtype == "f32" else lr.BF16

            def dev(x):
                if wl.dtype == "f32":
                    return torch.from_numpy(x).cuda()
                return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)

            a, b, g = dev(inp.a), dev(inp.b), dev(inp.g)
            del inp
            v = shape_variants()
            del v["walk"]
            res = measure(wl.B, wl.T, wl.D, dt, a, b, g, v)
            print(json.dumps({"sweep": "tiles", "workload": wname, "B": wl.B, "T": wl.T,
                              "D": wl.D, "dtype": wl.dtype, "steps": steps,
                              "best_fwd": best(res, "fwd_gbps"), "best_bwd": best(res, "bwd_gbps"),
                              **res}), flush=True)
            del a, b, g
            torch.cuda.empty_cache()


SWEEP_FAMILY_T = (8, 16, 32, 64, 128, 256, 1024)
SWEEP_COMPLEX_LANES = ((8, 8), (8, 32), (8, 128), (8, 512), (32, 8), (32, 32), (32, 128),
                       (32, 512), (64, 8), (64, 32), (64, 128), (64, 512))


def family_sweep_lines(args, lr, torch):
    """Short sequences of the complex and fused-transition scans, one JSON
    line per point (M = 2560, per-call HIP events with the Infinity Cache
    flushed before each call, the mean of `--steps` calls).

    complex: the tiled form (algo fused), the per-lane walk (seq) and the
      automatic choice, at constant work (B*T*M ~ 100M complex elements in
      bf16, 50M in fp32; T from 8 to 1024) and over the number of lanes B*M
      for T = 8, 32, 64 (B = 8 ... 512).
    samu: the fused-transition scan's tiles, its per-lane walk and the
      automatic choice at constant work (B*T*M ~ 84M bf16 elements, 42M
      fp32; T from 8 to 1024).
    Inputs are drawn on the device (a, b, grad_out ~ N(0, 0.5^2) per part for
    the complex scan; eta ~ N(0, 0.5^2), delta ~ N(0, 0.1^2), nu ~ U(0.005,
    0.5), theta ~ U(0.001, 3) for the fused-transition scan).  Rates are the
    interface bytes per second: complex forward 6*s*N + 8*B*M, backward
    10*s*N; fused-transition forward 4*s*N, backward 6*s*N."""
    import ctypes
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    flush = cache_flush(torch)
    steps = max(1, args.steps)
    L = lr.library()
    M = 2560

    def P(t):
        return t.data_ptr()

    def rate(nbytes, times):
        return round(nbytes / (sum(times) / len(times) * 1e-3) / 1e9, 1)

    def timed(f, bw, fb, bb):
        assert f() == 0 and bw() == 0
        torch.cuda.synchronize()
        tf, tb = cold_times(torch, stream, [f, bw], steps, flush)
        return {"fwd_gbps": rate(fb, tf), "bwd_gbps": rate(bb, tb),
                "fwd_us": round(sum(tf) / len(tf) * 1e3, 1),
                "bwd_us": round(sum(tb) / len(tb) * 1e3, 1)}

    dtypes = (("bf16", lr.BF16, torch.bfloat16, 2), ("f32", lr.F32, torch.float32, 4))
    if args.sweep == "complex":
        points = [(name, dt, tdt, s, T, max(1, int(round(2.0e8 * 2 / s / (T * M)))))
                  for name, dt, tdt, s in dtypes for T in SWEEP_FAMILY_T]
        points += [(name, dt, tdt, s, T, B) for name, dt, tdt, s in dtypes
                   for T, B in SWEEP_COMPLEX_LANES]
        for name, dt, tdt, s, T, B in points:
            ar, ai, br, bi, gr, gi = (torch.randn(B, T, M, device="cuda").mul_(0.5).to(tdt)
                                      for _ in range(6))
            o = [torch.empty_like(ar) for _ in range(6)]
            last = [torch.empty(B, M, device="cuda") for _ in range(2)]
            N = B * T * M
            res = {}
            for algo in ("fused", "seq", "auto"):
                op = lr.make_opts(algo=algo)
                f = lambda op=op: L.scan_complex_fwd(
                    P(ar), P(ai), P(br), P(bi), P(o[0]), P(o[1]), P(last[0]), P(last[1]), None,
                    None, B, T, M, dt, sh, ctypes.byref(op))
                bw = lambda op=op: L.scan_complex_bwd(
                    P(ar), P(ai), P(o[0]), P(o[1]), P(gr), P(gi), None, None, None, None, P(o[2]),
                    P(o[3]), P(o[4]), P(o[5]), None, None, B, T, M, dt, sh, ctypes.byref(op))
                res["walk" if algo == "seq" else ("tile" if algo == "fused" else "auto")] = timed(
                    f, bw, 6 * s * N + 8 * B * M, 10 * s * N)
            print(json.dumps({"sweep": "complex", "dtype": name, "B": B, "T": T, "M": M,
                              "lanes": B * M, "steps": steps, **res}), flush=True)
            del ar, ai, br, bi, gr, gi, o, last
            torch.cuda.empty_cache()
        return
    for name, dt, tdt, s in dtypes:
        for T in SWEEP_FAMILY_T:
            B = max(1, int(round(1.68e8 * 2 / s / (T * M))))
            eta = torch.randn(B, T, device="cuda").mul_(0.5).to(tdt)
            delta = torch.randn(B, T, device="cuda").mul_(0.1).to(tdt)
            nu = torch.empty(M, device="cuda").uniform_(0.005, 0.5).log_()
            th = torch.empty(M, device="cuda").uniform_(0.001, 3.0).log_()
            br, bi, gr, gi = (torch.randn(B, T, M, device="cuda").mul_(0.3).to(tdt)
                              for _ in range(4))
            o = [torch.empty_like(br) for _ in range(4)]
            last = [torch.empty(B, M, device="cuda") for _ in range(2)]
            grads = [torch.empty(B, T, device="cuda"), torch.empty(B, T, device="cuda"),
                     torch.empty(M, device="cuda"), torch.empty(M, device="cuda")]
            ctl = (P(eta), P(delta), P(nu), P(th))
            N = B * T * M
            res = {}
            for algo in ("fused", "seq", "auto"):
                op = lr.make_opts(algo=algo)
                f = lambda op=op: L.scan_samu_fwd(*ctl, P(br), P(bi), P(o[0]), P(o[1]),
                                                  P(last[0]), P(last[1]), None, None, B, T, M,
                                                  dt, sh, ctypes.byref(op))
                bw = lambda op=op: L.scan_samu_bwd(*ctl, P(o[0]), P(o[1]), P(gr), P(gi), None,
                                                   None, None, None, *(P(x) for x in grads),
                                                   P(o[2]), P(o[3]), None, None, B, T, M, dt, sh,
                                                   ctypes.byref(op))
                res["walk" if algo == "seq" else ("tile" if algo == "fused" else "auto")] = timed(
                    f, bw, 4 * s * N, 6 * s * N)
            print(json.dumps({"sweep": "samu", "dtype": name, "B": B, "T": T, "M": M,
                              "lanes": B * M, "steps": steps, **res}), flush=True)
            del eta, delta, br, bi, gr, gi, o, last, grads
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="default",
                    help="default: wide, long32, longseq, then masked (one line each, masked "
                         "last); or one of " + ", ".join(WORKLOAD_TEXT))
    ap.add_argument("--algo", default="auto")
    ap.add_argument("--fwd-chunk", type=int, default=0)
    ap.add_argument("--bwd-chunk", type=int, default=0)
    ap.add_argument("--fwd-width", type=int, default=0)
    ap.add_argument("--bwd-width", type=int, default=0)
    ap.add_argument("--mode", default="train", choices=["train", "prefill", "decode"],
                    help="train: forward + backward (the default line); prefill: the state-only "
                         "forward (reads a and b, writes last); decode: one scan_step per token "
                         "on the workload's [B, D] lanes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run kernels of known traffic (a 1 GiB device copy and the "
                         "read-2/write-1 streaming kernel on 3 x 256 MiB), the reference for "
                         "HBM byte counters")
    ap.add_argument("--sweep", choices=["lanes", "short", "tiles", "complex", "samu"],
                    help="print the dispatch measurements instead of the step: the per-lane "
                         "walk against the automatic choice over the number of lanes (lanes), "
                         "every tile shape on short sequences (short) or on the large "
                         "workloads (tiles), the complex scan's tiles against its walk on short "
                         "sequences (complex), the fused-transition scan's tiles against its walk "
                         "on short sequences (samu); one JSON line per point")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the scan is built and "
                                   "measured on a single MI355X (run with --gpus 1)"}))
        sys.exit(2)

    import torch

    import linear_recurrence_sequence_diag_amd as lr
    import workloads as W

    lr.library()  # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)

    if args.calibrate:
        # Kernels of known size: their HBM byte counters (FETCH_SIZE,
        # WRITE_SIZE) give the factors that turn counter readings into bytes.
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        y = torch.ones_like(x)
        z = torch.empty_like(x)
        ceil = StreamCeiling()
        sh = torch.cuda.current_stream().cuda_stream
        for _ in range(args.steps):
            ceil.run(1, 4, 0, [x, y], [z], x.numel() * 4, sh)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy and stream",
                          "copy": {"bytes_read": 4 * n, "bytes_written": 4 * n},
                          "stream_read2_write1": {"bytes_read": 2 * n, "bytes_written": n},
                          "repetitions": args.steps}))
        return

    if args.sweep in ("complex", "samu"):
        family_sweep_lines(args, lr, torch)
        return
    if args.sweep:
        sweep_lines(args, lr, torch, W)
        return

    if args.workload in W.COMPLEX_WORKLOADS:
        print(json.dumps(complex_line(args, W.COMPLEX_WORKLOADS[args.workload], lr, torch, W)),
              flush=True)
        return
    if args.workload in W.SAMU_WORKLOADS:
        print(json.dumps(samu_line(args, W.SAMU_WORKLOADS[args.workload], lr, torch, W)),
              flush=True)
        return
    names = DEFAULT_WORKLOADS if args.workload == "default" else (args.workload,)
    for i, name in enumerate(names):
        final = i == len(names) - 1
        print(json.dumps(train_line(args, name, lr, torch, W, 10.0 if final else 5.0)),
              flush=True)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
