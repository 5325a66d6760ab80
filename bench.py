#!/usr/bin/env python3
"""Benchmark of the selective spectral mixer core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

A step is one chunked prefill call over the largest single-GPU workload, the
128K-token DNA-like prefill (B=1, L=131072, K=24, m=4, P=64, Lc=128, bf16 v/gates,
fp32 clock and state), full tier K_T=24, inputs resident in HBM.  ``value`` is
tokens per second (B*L per step).  The same JSON line also carries
  * roofline: algorithmic bytes of one prefill call / its average duration (HIP
    events around each call on the launch stream) against 8 TB/s;
  * cpu_baseline: the CPU oracle (float32, -O3 -march=native, OpenMP over sequences)
    on the same workload, all host cores and one;
  * decode: the 24-layer batch-one decode workload (K=32, m=8, P=128, K_T=32),
    1024 steps replayed from a HIP graph, us/step and kernel roofline;
  * extra: tier sweeps of the three prefill workloads, the per-mode control form, and the
    decode at tiers K_T = 8, 16, 24 beside 32.
Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SLEEP_CYCLES = 200_000_000
# Summaries of rocprofv3 runs committed under profiles/: HBM bytes per launch from FETCH_SIZE
# and WRITE_SIZE passes (scaled by the same counters on a plain copy of known size), MFMA flops
# per launch, and the decode kernel's median duration.  Each records the SHA-256 of the kernel
# sources it was taken on and is used only while they still hash to it.
PREFILL_SOURCES = [os.path.join(ROOT, "selective_spectral_ssm_amd", "csrc", f)
                   for f in ("prefill_chunk_kernel.h", "prefill_chunk.hip", "prefill_wave.hip", "essh_internal.h")]
DECODE_SOURCES = [os.path.join(ROOT, "selective_spectral_ssm_amd", "csrc", f)
                  for f in ("decode.hip", "essh_internal.h")]
# The headline: the largest single-GPU workload (128K-token DNA-like prefill) at its full tier.
HEADLINE = (4, 24)
METRIC = "selective spectral scan prefill tokens/s + decode µs/step, % of HBM roofline"


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def to_dev(x):
    import numpy as np
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


MFMA_PEAK_TFLOPS = 2500.0   # dense bf16


def profile_text(name, key, sources):
    """A value recorded in profiles/<name>.md (a line "- key: `value`"), or None when the file
    is missing or was taken on kernel sources that no longer hash to its source_sha256."""
    try:
        text = open(os.path.join(ROOT, "profiles", name + ".md")).read()
    except OSError:
        return None
    kv = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
    if kv.get("source_sha256") != source_hash(sources):
        return None
    return kv.get(key)


def profile_value(name, key, sources):
    try:
        return float(profile_text(name, key, sources))
    except (TypeError, ValueError):
        return None


def copy_calibration(mib):
    """A plain elementwise copy (read N bytes, write N bytes) for the counter calibration."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 launches of neg over {mib} MiB fp32 (reads and writes {n * 4} bytes each)")


def copy_bandwidth(mib=1024, reps=10):
    """Bytes read + written per second by a plain elementwise copy over mib MiB:
    the bandwidth an ideal streaming kernel reaches on this device."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) * 1e-3 / reps
    del src, dst
    return 2 * n * 4 / sec / 1e9


def copy_time_us(total_bytes, reps=50):
    """Mean time of a plain elementwise copy that reads total_bytes/2 and writes
    total_bytes/2: what moving a kernel's bytes costs at this size, launch
    ramp-up and drain included."""
    import torch
    n = max(1, total_bytes // 8)
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(SLEEP_CYCLES // 4)
    for a, b in evs:
        a.record()
        torch.neg(src, out=dst)
        b.record()
    torch.cuda.synchronize()
    return statistics.mean(a.elapsed_time(b) for a, b in evs) * 1e3


def time_launches(fn, steps, warmup):
    """Returns (ms per step over the whole timed region, mean and median ms per launch).

    The timed region is `steps` back-to-back launches with nothing between them;
    the per-launch durations come from a second pass of `steps` launches, each
    bracketed by HIP events on the launch stream (events between launches add
    a little time of their own, so they stay out of the timed region)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # Keep the GPU busy while the host enqueues the timed launches, so that the
    # events measure back-to-back GPU execution and not host submission speed.
    torch.cuda._sleep(SLEEP_CYCLES)
    t0.record(s)
    for _ in range(steps):
        fn()
    t1.record(s)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda._sleep(SLEEP_CYCLES)
    for a, b in ev:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return total, statistics.mean(per), statistics.median(per)


_CACHE = {}


def workload_inputs(widx, per_mode=False):
    from selective_spectral_ssm_amd import inputs as I
    key = (widx, per_mode)
    if key not in _CACHE:
        _CACHE.clear()
        w = I.workload(widx)
        inp = I.make_prefill_inputs(w, per_mode=per_mode)
        d = {k: to_dev(inp[k]) for k in ("v", "delta", "g_w", "g_r", "rho", "theta", "c")}
        _CACHE[key] = (w, inp, d)
    return _CACHE[key]


def prefill_case(widx, K_T, steps, warmup, per_mode=False):
    """One workload at tier K_T; per_mode: clock and gates per mode ([B, L, K, m])."""
    from selective_spectral_ssm_amd import essh, sizes
    w, inp, d = workload_inputs(widx, per_mode)
    call = essh.Prefill(d["v"], d["delta"], d["g_w"], d["g_r"], d["rho"], d["theta"], d["c"],
                        K_T=K_T, Lc=w.Lc, want_state=True)
    ms_step, ms_launch, ms_med = time_launches(call.run, steps, warmup)
    call.check()                 # a look-back wait that ran out would have made the outputs invalid
    nbytes = sizes.prefill_bytes(w.B, w.L, K_T, w.m, w.P, w.io, write_state=True, per_mode=per_mode)
    return dict(workload=w.name, K_T=K_T, ms_per_step=ms_step, us_per_launch=ms_launch * 1e3,
                us_per_launch_median=ms_med * 1e3,
                tokens_per_s=w.B * w.L / (ms_step * 1e-3),
                kernel_tokens_per_s=w.B * w.L / (ms_launch * 1e-3),
                alg_bytes=nbytes, achieved_GBs=nbytes / (ms_launch * 1e-3) / 1e9), w, inp


def decode_case(K_T, n_steps=1024, reps=3, context=2048):
    import torch
    from selective_spectral_ssm_amd import essh, inputs as I, sizes
    w = I.workload(3)
    key = ("decode", n_steps, context)
    if key not in _CACHE:
        log(f"decode: drawing inputs ({w.layers} layers, context {context}, {n_steps} steps)")
        _CACHE.clear()
        _CACHE[key] = I.make_decode_inputs(w, n_steps=n_steps, context=context)
    dec = _CACHE[key]
    NL = w.layers
    rho, theta, c = to_dev(dec["rho"]), to_dev(dec["theta"]), to_dev(dec["c"])
    state = torch.zeros((NL, 1, w.K, w.m, 2, w.P), device="cuda")
    for l in range(NL):
        _, st = essh.prefill(to_dev(dec["ctx_v"][l]), to_dev(dec["ctx_delta"][l]), to_dev(dec["ctx_g_w"][l]),
                             to_dev(dec["ctx_g_r"][l]), rho[l], theta[l], c[l], K_T=K_T, Lc=64)
        state[l] = st
    sv, sd, sgw, sgr = (to_dev(dec[k]) for k in ("step_v", "step_delta", "step_g_w", "step_g_r"))
    y = torch.empty((n_steps, NL, 1, w.K, w.P), dtype=torch.bfloat16, device="cuda")
    dims = essh.make_dims(1, 1, w.K, w.m, w.P, K_T, 0, False, "bf16")
    state0 = state.clone()

    def step(s):
        rc = essh.essh_mixer_decode_step(NL, dims, sv[s], sd[s], sgw[s], sgr[s], rho, theta, c, None, state, y[s])
        assert rc == 0

    # kernel duration: HIP events around each launch (eager)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    for s in range(32):
        step(s)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    torch.cuda._sleep(SLEEP_CYCLES)   # GPU busy while the host enqueues (see time_launches)
    for s in range(n_steps):
        ev[s][0].record(cur)
        step(s)
        ev[s][1].record(cur)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) * 1e3 for a, b in ev]
    # whole-step wall time: the 1024-step loop captured once in a HIP graph, replayed
    state.copy_(state0)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step(0)                      # warm the capture stream
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for s in range(n_steps):
            step(s)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        state.copy_(state0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) * 1e6 / n_steps)
    nbytes = sizes.decode_bytes(NL, 1, K_T, w.m, w.P, "bf16")
    kmean = statistics.mean(per)
    # the decode kernel's own median duration, from the committed rocprofv3 kernel trace
    k_rocprof = profile_value("kernel_trace_decode_mixer1p5b", f"median_us_kt{K_T}", DECODE_SOURCES)
    # Achieved bandwidth from the graph replay: one kernel per step back to back, so the
    # per-step time is the kernel plus the gap to the next one.  Events around each
    # eager launch add their own overhead to a kernel this short and read higher.
    us_step = statistics.median(times)
    return dict(workload=w.name, layers=NL, K_T=K_T, steps=n_steps, copy_same_bytes_us=copy_time_us(nbytes),
                us_per_step_graph=us_step, us_per_step_graph_all=times,
                us_per_kernel_mean=kmean, us_per_kernel_median=statistics.median(per),
                us_per_kernel_rocprof_median=k_rocprof,
                frac_of_hbm_peak_kernel=None if k_rocprof is None else nbytes / (k_rocprof * 1e-6) / 1e9 / HBM_PEAK_GBS,
                alg_bytes_per_step=nbytes, achieved_GBs=nbytes / (us_step * 1e-6) / 1e9,
                frac_of_hbm_peak=nbytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBS,
                achieved_GBs_eager_events=nbytes / (kmean * 1e-6) / 1e9)


def decode_fused_case(K_T, steps=20, warmup=3):
    """The fused decode step with projections at the decode workload's layer shape (24 layers,
    B=1, K=32, m=8, P=128, d = K P = 4096): random-init bf16 weights drawn on the GPU from a
    seeded generator; events around `steps` back-to-back steps (two launches each)."""
    import torch
    from selective_spectral_ssm_amd import essh, inputs as I, sizes
    w = I.workload(3)
    NL, B, K, m, P = w.layers, w.B, w.K, w.m, w.P
    D = K * P
    key = ("fused",)
    if key not in _CACHE:
        _CACHE.clear()
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed)

        def randn(*shape, std=1.0):
            return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)

        t = dict(u=randn(NL, B, D), w_in=randn(NL, K, P, D, std=D ** -0.5),
                 w_ctl=randn(NL, K, m, 3, D, std=D ** -0.5), w_out=randn(NL, D, K, P, std=(K * P) ** -0.5),
                 beta=torch.rand(NL, K, generator=g, device="cuda") * 2 - 0.5,
                 b_ctl=torch.randn(NL, K, m, 3, generator=g, device="cuda") - torch.tensor([0., 0., 2.], device="cuda"),
                 rho=torch.rand(NL, K, m, generator=g, device="cuda") * (w.rho_hi - w.rho_lo) + w.rho_lo,
                 theta=torch.rand(NL, K, m, generator=g, device="cuda") * 3.141592653589793,
                 c=torch.randn(NL, K, m, 2, generator=g, device="cuda") * (2 * m) ** -0.5,
                 state=torch.randn(NL, B, K, m, 2, P, generator=g, device="cuda"))
        _CACHE[key] = t
    t = _CACHE[key]
    z = torch.empty(NL, B, K, P, device="cuda")
    y = torch.empty(NL, B, D, device="cuda")
    dims = essh.make_dims(B, 1, K, m, P, K_T, 0, False, "bf16")

    def step():
        rc = essh.essh_decode_fused_step(NL, dims, D, t["u"], t["w_in"], t["beta"], 1e-5, t["w_ctl"], t["b_ctl"],
                                         t["rho"], t["theta"], t["c"], None, t["w_out"], t["state"], z, y)
        assert rc == 0

    _, ms_launch, ms_med = time_launches(step, steps, warmup)
    nbytes = sizes.decode_fused_bytes(NL, B, K_T, m, P, D, "bf16")
    us = ms_launch * 1e3
    return dict(layers=NL, d_model=D, K_T=K_T, us_per_step=us, us_per_step_median=ms_med * 1e3,
                alg_bytes_per_step=nbytes, achieved_GBs=nbytes / (us * 1e-6) / 1e9,
                frac_of_hbm_peak=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                tflops=sizes.decode_fused_flops(NL, B, K_T, m, P, D) / (us * 1e-6) / 1e12)


def backward_case(widx, K_T, steps, warmup):
    """The backward pass of one prefill workload at tier K_T (entering state, zero-lag
    coefficients and the final state's gradient all given): dy ~ N(0,1) and the extra inputs are
    drawn on the GPU from a seeded generator."""
    import torch
    from selective_spectral_ssm_amd import essh, sizes
    w, inp, d = workload_inputs(widx)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 1000)
    B, L, K, P, m = w.B, w.L, w.K, w.P, w.m
    dy = torch.randn(B, L, K, P, generator=g, device="cuda").to(d["v"].dtype)
    s_in = torch.randn(B, K, m, 2, P, generator=g, device="cuda")
    dso = torch.randn(B, K, m, 2, P, generator=g, device="cuda")
    zl = torch.rand(K, m, generator=g, device="cuda")
    call = essh.PrefillBackward(d["v"], d["delta"], d["g_w"], d["g_r"], d["rho"], d["theta"], d["c"], dy,
                                K_T=K_T, state_in=s_in, dstate_out=dso, zl=zl)
    ms_step, ms_launch, ms_med = time_launches(call.run, steps, warmup)
    nbytes = sizes.backward_bytes(B, L, K_T, m, P, w.io)
    return dict(workload=w.name, K_T=K_T, us_per_call=ms_launch * 1e3, us_per_call_median=ms_med * 1e3,
                ms_per_step=ms_step, tokens_per_s=B * L / (ms_step * 1e-3), alg_bytes=nbytes,
                achieved_GBs=nbytes / (ms_launch * 1e-3) / 1e9,
                frac_of_hbm_peak=nbytes / (ms_launch * 1e-3) / 1e9 / HBM_PEAK_GBS,
                workspace_MiB=call.ws_bytes / 2 ** 20)


def _lscpu_model():
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


def cpu_baseline(inp, w, K_T, runs=5):
    """The CPU oracle timed on this host: the oracle's C source built
    as float32 with -O3 -march=native for this host, OpenMP over the independent (batch row,
    channel) sequences on every host core, median of `runs` runs after one warm-up; the same
    on one thread; and the decode step (24 layers) on all cores.  A reported baseline only."""
    import numpy as np

    import oracle
    from selective_spectral_ssm_amd.inputs import as_f64
    so = oracle.build_native(os.path.join(ROOT, "oracle", "_build"))
    run = oracle.make_prefill(so_path=so, precision="f32")
    ncores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    x = dict(v=as_f64(inp["v"], w.io).astype(np.float32), delta=inp["delta"],
             g_w=as_f64(inp["g_w"], w.io).astype(np.float32), g_r=as_f64(inp["g_r"], w.io).astype(np.float32),
             rho=inp["rho"], theta=inp["theta"], c=inp["c"])

    def timed(nthreads, kt):
        ts = []
        for i in range(runs + 1):
            t0 = time.perf_counter()
            run(**x, K_T=kt, nthreads=nthreads)
            if i > 0:                       # the first run is the warm-up
                ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    med = timed(ncores, K_T)
    cores = oracle.threads_used("f32", so_path=so)
    # one thread: a bounded sample, the first kt1 of the K_T channels (every channel is the same
    # amount of work), scaled to the whole tier
    kt1 = max(1, min(K_T, (2 * w.B * 131072) // (w.B * w.L) if w.L else K_T))
    med1 = timed(1, kt1) * K_T / kt1
    nb = w.B * w.L
    res = dict(value=nb / med, unit="tokens/s", cores=cores, kind="oracle",
               sample=f"whole {w.name} workload (B={w.B}, L={w.L}, K_T={K_T}), float32 oracle built -O3 "
                      f"-march=native, OpenMP over (b, k) sequences, median of {runs} runs after 1 warm-up",
               cpu_model=_lscpu_model(), nproc=ncores, seconds_per_run=med,
               single_thread=dict(value=nb / med1, cores=1, seconds_per_run=med1,
                                  sample=f"one thread, the first {kt1} of the {K_T} channels of every batch row "
                                         f"(median of {runs} runs after 1 warm-up), scaled by {K_T}/{kt1}"))
    # decode: the 24-layer step (K_T = 32) on all cores, over a bounded number of steps
    from selective_spectral_ssm_amd import inputs as I
    wd = I.workload(3)
    n_steps = 16
    dec = I.make_decode_inputs(wd, n_steps=n_steps + 1, context=1)
    st = np.zeros((wd.layers, 1, wd.K, wd.m, 2, wd.P), np.float32)

    def dstep(s, st):
        ys, sts = [], []
        for l in range(wd.layers):
            y, s2 = run(as_f64(dec["step_v"][s, l][:, None], "bf16").astype(np.float32),
                        dec["step_delta"][s, l][:, None], as_f64(dec["step_g_w"][s, l][:, None], "bf16"),
                        as_f64(dec["step_g_r"][s, l][:, None], "bf16"), dec["rho"][l], dec["theta"][l],
                        dec["c"][l], state_in=st[l], nthreads=ncores)
            sts.append(s2)
        return np.stack(sts)
    st = dstep(0, st)                        # warm-up
    t0 = time.perf_counter()
    for s in range(1, n_steps + 1):
        st = dstep(s, st)
    res["decode_us_per_step"] = (time.perf_counter() - t0) / n_steps * 1e6
    res["decode_sample"] = (f"{n_steps} steps of the 24-layer decode (K=K_T=32, m=8, P=128, B=1), "
                            f"float32 oracle on {ncores} threads, after 1 warm-up step")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the tier sweeps")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain copy of this many MiB (counter calibration)")
    ap.add_argument("--workload", type=int, default=HEADLINE[0],
                    help="prefill workload of the main line (profiling runs; default: the headline)")
    ap.add_argument("--kt", type=int, default=HEADLINE[1], help="its tier K_T")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode at every tier (profiling runs); prints the decode JSON")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the prefill backward of --workload at --kt (profiling runs); prints its JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_spectral_ssm_amd import essh, sizes
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    essh.lib()   # fail loudly if the HIP library is not built
    if args.copy_mib > 0:
        copy_calibration(args.copy_mib)

    from selective_spectral_ssm_amd import inputs as I
    if args.decode_only:
        out = []
        for kt in I.WORKLOADS[3].tiers:
            log(f"decode: 24 layers K_T={kt}")
            out.append(decode_case(kt))
        fz = [decode_fused_case(kt) for kt in (8, 16, 24, 32)]
        print(json.dumps({"decode_tiers": out, "decode_fused": fz}))
        return
    widx, KT = args.workload, args.kt
    if args.backward_only:
        log(f"backward: workload {widx} K_T={KT}")
        print(json.dumps({"backward": backward_case(widx, KT, args.steps, args.warmup)}))
        return
    wname = I.WORKLOADS[widx].name
    log(f"prefill: {wname} K_T={KT}")
    main_res, w, inp = prefill_case(widx, KT, args.steps, args.warmup)
    tag = f"prefill_{wname.replace('_prefill', '')}_kt{KT}"
    traffic = profile_value("hbm_traffic_" + tag, "hbm_bytes_per_launch", PREFILL_SOURCES)
    mfma = profile_value("mfma_" + tag, "mfma_flops_per_launch", PREFILL_SOURCES)
    # the launches of one prefill call and the sum of their average durations in the
    # committed kernel trace of this command (rocprofv3), beside the live HIP-event figure
    launches = profile_text("kernel_trace_" + tag, "launches", PREFILL_SOURCES)
    trace_us = profile_value("kernel_trace_" + tag, "sum_avg_us", PREFILL_SOURCES)
    copy_gbs = copy_bandwidth()
    log(f"plain copy: {copy_gbs:.0f} GB/s (read + write)")
    us = main_res["us_per_launch"]
    res = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "K": w.K, "K_T": KT, "m": w.m, "P": w.P,
                   "Lc": w.Lc, "io": w.io, "state": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": "every launch of one essh_mixer_prefill call" + (f": {launches}" if launches else ""),
                     "rocprof_sum_avg_us": trace_us,
                     "achieved": main_res["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": main_res["achieved_GBs"] / HBM_PEAK_GBS,
                     "traffic": None if traffic is None else traffic / (us * 1e-6) / 1e9,
                     "traffic_bytes_per_launch": traffic,
                     "mfma": None if mfma is None else {
                         "flops_per_launch": mfma, "achieved": mfma / (us * 1e-6) / 1e12,
                         "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": mfma / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS},
                     "alg_bytes_per_launch": main_res["alg_bytes"],
                     "copy_GBs": copy_gbs, "frac_of_copy": main_res["achieved_GBs"] / copy_gbs,
                     "copy_same_bytes_us": copy_time_us(main_res["alg_bytes"]),
                     "us_per_launch": us},
    }
    if not args.no_decode:
        log("decode: 24 layers K_T=32")
        res["decode"] = decode_case(32)
        fz = []
        for kt in (8, 16, 24, 32):
            log(f"fused decode with projections: 24 layers K_T={kt}")
            fz.append(decode_fused_case(kt))
        res["decode_fused"] = fz
    if not args.no_extra:
        extra = []
        for wi in (1, 2, 4):
            for kt in I.WORKLOADS[wi].tiers:
                if (wi, kt) == (widx, KT):
                    r = main_res
                else:
                    log(f"tier sweep: workload {wi} K_T={kt}")
                    r, _, _ = prefill_case(wi, kt, max(10, args.steps // 4), 5)
                extra.append({k: r[k] for k in ("workload", "K_T", "us_per_launch", "kernel_tokens_per_s",
                                                "achieved_GBs")})
                extra[-1]["frac"] = r["achieved_GBs"] / HBM_PEAK_GBS
        res["prefill_tiers"] = extra
        pm = []
        for wi, kt in ((1, 24), (2, 32), (2, 8)):
            log(f"per-mode controls: workload {wi} K_T={kt}")
            r, _, _ = prefill_case(wi, kt, max(10, args.steps // 4), 5, per_mode=True)
            pm.append({k: r[k] for k in ("workload", "K_T", "us_per_launch", "kernel_tokens_per_s", "achieved_GBs")})
            pm[-1]["frac"] = r["achieved_GBs"] / HBM_PEAK_GBS
        res["prefill_per_mode"] = pm
        if not args.no_decode:
            dt = []
            for kt in (8, 16, 24):
                log(f"decode tier sweep: K_T={kt}")
                r = decode_case(kt)
                dt.append({k: r[k] for k in ("K_T", "us_per_step_graph", "alg_bytes_per_step", "achieved_GBs",
                                             "frac_of_hbm_peak", "us_per_kernel_rocprof_median",
                                             "frac_of_hbm_peak_kernel")})
            dt.append({k: res["decode"][k] for k in dt[0]})
            res["decode_tiers"] = dt
    if not args.no_extra:
        bw = []
        for wi in (1, 2, 4):
            kt = I.WORKLOADS[wi].tiers[-1]
            log(f"prefill backward: workload {wi} K_T={kt}")
            bw.append(backward_case(wi, kt, max(10, args.steps // 10), 3))
        res["prefill_backward"] = bw
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(inp, w, KT)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
