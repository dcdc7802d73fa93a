#!/usr/bin/env python3
"""Benchmark of the fused Q+K layerwise RMSNorm on one MI355X.

One step = one fused call (every stage of the path: shard partials, scalar
exchange and combine, x*gamma, final scaling) over the prefill workload:
T=16384 tokens, Q and K width 5120, bf16, 2 logical shards, inputs resident
in HBM. Prints ONE JSON line on stdout; progress goes to stderr.

Every input of every leg is drawn and copied to the device before the first
leg is timed. Each leg then runs its own kernel untimed until the per-call time
of consecutive batches agrees (the "preroll", reported per leg: the GPU's clocks
ramp under load and would otherwise bias a short run), then --warmup untimed
calls, then exactly --steps timed calls between HIP events on the launch stream.

Besides the headline (GB/s of algorithmic bytes), the line carries:
  decode      -- the T=64 decode workload: device and host-visible us per call
  copy        -- a plain copy of the same bytes (achievable-bandwidth ceiling)
  split       -- the three-kernel split path on the same workload
  roofline    -- the fused kernel against MI355X peak HBM bandwidth
  cpu_baseline-- the fp64 oracle timed on this host's cores on a sample
  cpu_host    -- the host CPU model and the oracle's rate on one core
  tiny        -- the tiny fp32 workload: fp64 oracle ms and device us per call

  e4m3        -- FP8-E4M3 activations (bf16 gamma) on the prefill shape with bf16
                 and with E4M3 outputs, each against the HBM roofline and a ceiling
                 moving the same bytes, and the decode shape in us per call
  layernorm   -- LayerNorm (two additive shard statistics, gamma and beta) on the
                 prefill shape against the HBM roofline and the copy ceiling, and
                 the decode shape
  headwise    -- headwise QK-Norm (one factor per head of 128 columns) on the
                 prefill shape against the HBM roofline and the copy ceiling
  gqa         -- the GQA-shaped workload (Q width 5120, K width 1024, 4 shards)
                 against the HBM roofline and a copy of the same tensors

Modes: ``--pmc`` runs only the kernels whose counters are collected
(fused prefill in bf16, in E4M3->bf16, in E4M3->E4M3 and as LayerNorm, headwise
prefill, GQA, and the copy of known size), for rocprofv3 --pmc runs.
"""
import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, 8 TB/s
METRIC = "fused Q+K layerwise RMSNorm HBM GB/s (% of peak) at T=16384; decode µs at T=64"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_SUMMARY = os.path.join(PROFILES, "fused_prefill_T16384_traffic.txt")
TRAFFIC_SUMMARY_E4M3 = os.path.join(PROFILES, "fused_prefill_e4m3_T16384_traffic.txt")
TRAFFIC_SUMMARY_LN = os.path.join(PROFILES, "fused_layernorm_prefill_T16384_traffic.txt")
TRAFFIC_SUMMARY_E4M3_E4M3 = os.path.join(PROFILES, "fused_prefill_e4m3_to_e4m3_T16384_traffic.txt")
TRAFFIC_SUMMARY_HW = os.path.join(PROFILES, "headwise_prefill_T16384_traffic.txt")
TRAFFIC_SUMMARY_GQA = os.path.join(PROFILES, "fused_gqa_T8192_traffic.txt")
# the headwise kernel is one-shot (no planner): its launch is named by its shape
HEADWISE_PLAN = {"kernel": "headwise", "vectors_per_head": 16, "threads": 256}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def read_traffic(path, plan):
    """HBM bytes per launch from a committed counter summary, if it is current: taken
    on the same device code and with the launch plan this run uses."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    from layerwise_qk_norm_amd.profiling import kernel_source_sha, plan_line
    if kv.get("kernel_source_sha") != kernel_source_sha() or kv.get("plan") != plan_line(plan):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed(fn, steps, stream, torch, first=0):
    """Average ms per call of ``fn`` over ``steps`` back-to-back calls
    ``fn(first), ..., fn(first + steps - 1)``, between HIP events recorded on the
    stream the calls are issued on."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        fn(first + i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


class Leg:
    """One timed kernel: preroll until stable, ``warmup`` untimed calls, then
    ``steps`` timed calls. Call indices keep counting across the three stages,
    so rotating buffer sets stay in rotation."""

    def __init__(self, fn, stream, torch):
        self.fn, self.stream, self.torch = fn, stream, torch
        self.calls = 0
        self.preroll = None

    def run_preroll(self, batch=50, min_calls=300, max_calls=6000, tol=0.01):
        """Batches of ``batch`` calls until the last three batch averages lie within
        ``tol`` of each other (at least ``min_calls``, at most ``max_calls`` calls)."""
        per, t0 = [], time.perf_counter()
        while True:
            per.append(timed(self.fn, batch, self.stream, self.torch, self.calls))
            self.calls += batch
            last = per[-3:]
            if self.calls >= min_calls and len(last) == 3 and max(last) - min(last) <= tol * min(last):
                stable = True
                break
            if self.calls >= max_calls:
                stable = False
                break
        self.preroll = {"calls": self.calls, "s": round(time.perf_counter() - t0, 3),
                        "first_batch_us_per_call": round(per[0] * 1e3, 3),
                        "last_batches_us_per_call": [round(p * 1e3, 3) for p in per[-3:]],
                        "stable": stable}
        return self.preroll

    def measure(self, warmup, steps):
        for _ in range(warmup):
            self.fn(self.calls)
            self.calls += 1
        ms = timed(self.fn, steps, self.stream, self.torch, self.calls)
        self.calls += steps
        return ms


def timed_leg(fn, args, stream, torch, preroll=True):
    leg = Leg(fn, stream, torch)
    if preroll:
        leg.run_preroll()
    ms = leg.measure(args.warmup, args.steps)
    return ms, leg.preroll


def upload_sets(w, d, torch, sets):
    """``sets`` device copies of a workload's (q, k, out_q, out_k), plus its gammas."""
    from layerwise_qk_norm_amd import inputs
    dev = "cuda:0"
    gq, gk = inputs.to_device(d["gamma_q"], dev, torch), inputs.to_device(d["gamma_k"], dev, torch)
    odt = {"bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.float8_e4m3fn}[w.out]
    bufs = []
    for _ in range(sets):
        q = inputs.to_device(d["q"], dev, torch)
        k = inputs.to_device(d["k"], dev, torch)
        bufs.append((q, k, torch.empty(q.shape, dtype=odt, device=dev),
                     torch.empty(k.shape, dtype=odt, device=dev)))
    return gq, gk, bufs


def roofline(nbytes, ms, traffic):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}


def ceiling(kind, moved_bytes, ms, fused_ms, preroll):
    """A kernel moving the fused kernel's streaming bytes (Q and K read, outputs
    written) with the simplest access pattern, and the fused kernel's fraction of it."""
    return {"kind": kind, "bytes": moved_bytes, "ms": round(ms, 5),
            "GBs": round(moved_bytes / (ms * 1e-3) / 1e9, 1),
            "fused_frac_of_ceiling": round(ms / fused_ms, 4), "preroll": preroll}


def skeleton(args, stream, torch, bufs, w, fmt, moved_bytes, fused_ms):
    """The fused call's own launch plan run as a copy (no arithmetic, no exchange) on
    the leg's buffer sets: what the persistent streaming structure itself moves, and
    the fused kernel's fraction of it."""
    from layerwise_qk_norm_amd import ops

    def run(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.bench_skeleton(q, k, oq, ok, w.n_shards, fmt)

    ms, pre = timed_leg(run, args, stream, torch)
    return {"kind": "the fused call's launch plan as a copy (no arithmetic, no exchange)",
            "bytes": moved_bytes, "ms": round(ms, 5), "GBs": round(moved_bytes / (ms * 1e-3) / 1e9, 1),
            "fused_frac_of_skeleton": round(ms / fused_ms, 4), "preroll": pre}


# ---------------------------------------------------------------- legs

def leg_layernorm(args, torch, stream, prep):
    from layerwise_qk_norm_amd import ops
    out = {}
    w, par, bufs = prep["ln_prefill"]

    def fused(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.layernorm_fwd(q, k, par["gamma_q"], par["gamma_k"], w.n_shards, w.eps,
                          beta_q=par["beta_q"], beta_k=par["beta_k"], out_q=oq, out_k=ok)

    ms, pre = timed_leg(fused, args, stream, torch)
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("LayerNorm prefill reported an exchange timeout")
    nbytes = w.algorithmic_bytes()
    plan = ops.current_plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
    out["prefill"] = {
        "workload": f"T={w.T}, Q and K width {w.Hq}, bf16, gamma and beta, {w.n_shards} logical shards",
        "algorithmic_bytes": nbytes, "ms": round(ms, 5), "preroll": pre, "plan": plan,
        "roofline": roofline(nbytes, ms, read_traffic(TRAFFIC_SUMMARY_LN, plan)),
        "ceiling": ceiling("copy of the same bytes (the bf16 prefill copy leg)",
                           prep["copy_bytes"], prep["copy_ms"], ms, "shared with the copy leg"),
        "skeleton": skeleton(args, stream, torch, bufs, w, "ln_bf16", prep["copy_bytes"], ms)}
    wd, t, (oq, ok) = prep["ln_decode"]

    def dec(_):
        ops.layernorm_fwd(t["q"], t["k"], t["gamma_q"], t["gamma_k"], wd.n_shards, wd.eps,
                          beta_q=t["beta_q"], beta_k=t["beta_k"], out_q=oq, out_k=ok)

    for i in range(50):
        dec(i)
    us = timed(dec, 1000, stream, torch) * 1e3
    # a prepared call (validated once) issues back to back at the device rate
    pcall = ops.prepare_layernorm_fwd(t["q"], t["k"], t["gamma_q"], t["gamma_k"], wd.n_shards,
                                      wd.eps, beta_q=t["beta_q"], beta_k=t["beta_k"], out_q=oq,
                                      out_k=ok)
    for i in range(50):
        pcall()
    us_prep = timed(lambda _: pcall(), 1000, stream, torch) * 1e3
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("LayerNorm decode reported an exchange timeout")
    out["decode"] = {"workload": "T=64, Q and K width 4096, bf16, 4 logical shards",
                     "python_back_to_back_us_per_call": round(us, 2),
                     "prepared_back_to_back_us_per_call": round(us_prep, 2)}
    return out


def leg_gqa(args, torch, stream, prep):
    """The GQA-shaped workload (T=8192, Q width 5120, K width 1024, 4 logical shards).
    One call moves 201 MB, less than the 256 MB Infinity Cache, so three buffer sets
    rotate (604 MB) and every call streams from HBM; the copy ceiling rotates the
    same three sets."""
    from layerwise_qk_norm_amd import ops
    w, gq, gk, bufs = prep["gqa"]

    def fused(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=oq, out_k=ok)

    def copy(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.bench_copy(q, k, oq, ok)

    ms, pre = timed_leg(fused, args, stream, torch)
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("GQA workload reported an exchange timeout")
    copy_ms, copy_pre = timed_leg(copy, args, stream, torch)
    nbytes = w.algorithmic_bytes()
    moved = nbytes - (w.Hq + w.Hk) * w.elem_bytes
    plan = ops.current_plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
    return {"workload": f"T={w.T}, Q width {w.Hq}, K width {w.Hk}, bf16, {w.n_shards} logical shards",
            "algorithmic_bytes": nbytes, "ms": round(ms, 5), "preroll": pre, "plan": plan,
            "roofline": roofline(nbytes, ms, read_traffic(TRAFFIC_SUMMARY_GQA, plan)),
            "ceiling": ceiling("copy of Q and K, three rotating sets", moved, copy_ms, ms, copy_pre),
            "skeleton": skeleton(args, stream, torch, bufs, w, "bf16", moved, ms)}


def leg_headwise(args, torch, stream, prep):
    """Headwise QK-Norm (one factor per head of 128 columns) on the prefill shape."""
    from layerwise_qk_norm_amd import ops
    w, gq, gk, bufs = prep["headwise"]

    def fused(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.headwise_fwd(q, k, gq, gk, w.head_dim, w.eps, out_q=oq, out_k=ok)

    ms, pre = timed_leg(fused, args, stream, torch)
    nbytes = w.algorithmic_bytes()
    return {"prefill": {
        "workload": f"T={w.T}, Q and K width {w.Hq} ({w.Hq // w.head_dim} heads of {w.head_dim}), bf16",
        "algorithmic_bytes": nbytes, "ms": round(ms, 5), "preroll": pre,
        "roofline": roofline(nbytes, ms, read_traffic(TRAFFIC_SUMMARY_HW, HEADWISE_PLAN)),
        "ceiling": ceiling("copy of the same bytes (the bf16 prefill copy leg)",
                           prep["copy_bytes"], prep["copy_ms"], ms, "shared with the copy leg")}}


def leg_e4m3(args, torch, stream, prep):
    """FP8-E4M3 activations: prefill with bf16 and with E4M3 outputs, decode. Three
    buffer sets rotate (the inputs of one call are 168 MB, inside the Infinity Cache);
    each output format has a ceiling moving its bytes over the same sets: the
    widening copy (1 byte read, 2 written) for bf16 outputs, the plain copy for E4M3."""
    from layerwise_qk_norm_amd import ops
    out = {}
    for key in ("prefill_to_bf16", "prefill_to_e4m3"):
        w, gq, gk, bufs = prep[key]

        def fused(i):
            q, k, oq, ok = bufs[i % len(bufs)]
            ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=oq, out_k=ok)

        if w.out == "bf16":
            def ceil_fn(i):
                q, k, oq, ok = bufs[i % len(bufs)]
                ops.bench_widen(q.view(torch.uint8), k.view(torch.uint8), oq, ok)
            kind = "widening copy (each E4M3 byte read, a 16-bit word written), three rotating sets"
        else:
            def ceil_fn(i):
                q, k, oq, ok = bufs[i % len(bufs)]
                ops.bench_copy(q.view(torch.uint8), k.view(torch.uint8), oq.view(torch.uint8),
                               ok.view(torch.uint8))
            kind = "copy of the same bytes, three rotating sets"

        ms, pre = timed_leg(fused, args, stream, torch)
        if ops.check_fault() != ops.QKN_OK:
            raise RuntimeError("E4M3 prefill reported an exchange timeout")
        cms, cpre = timed_leg(ceil_fn, args, stream, torch)
        nbytes = w.algorithmic_bytes()
        moved = nbytes - (w.Hq + w.Hk) * 2
        plan = ops.current_plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
        traffic = read_traffic(TRAFFIC_SUMMARY_E4M3 if w.out == "bf16" else TRAFFIC_SUMMARY_E4M3_E4M3, plan)
        out[key] = {
            "workload": f"T={w.T}, Q and K width {w.Hq}, E4M3 in, bf16 gamma, {w.out} out, "
                        f"{w.n_shards} logical shards",
            "algorithmic_bytes": nbytes, "ms": round(ms, 5), "preroll": pre, "plan": plan,
            "roofline": roofline(nbytes, ms, traffic),
            "ceiling": ceiling(kind, moved, cms, ms, cpre),
            "skeleton": skeleton(args, stream, torch, bufs, w, w.fmt, moved, ms)}
    wd, dgq, dgk, (q, k, oq, ok) = prep["decode_e4m3"]
    ops.bench_fused(q, k, dgq, dgk, wd.n_shards, wd.eps, oq, ok, 200)
    reps = 2000
    c_us = timed(lambda _: ops.bench_fused(q, k, dgq, dgk, wd.n_shards, wd.eps, oq, ok, reps),
                 1, stream, torch) * 1e3 / reps
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("E4M3 decode reported an exchange timeout")
    out["decode"] = {"workload": "T=64, Q and K width 4096, E4M3 in and out, 4 logical shards",
                     "device_us_per_call": round(c_us, 2)}
    return out


def leg_tiny(torch, stream, prep):
    """The tiny fp32 workload (T=8, width 256, 2 shards): the fp64 oracle's time per
    call in ms on one core, and the device's time per call issued from C."""
    from layerwise_qk_norm_amd import ops
    from oracle import oracle
    w, d, (q, k, gq, gk, oq, ok) = prep["tiny"]
    reps = 200
    t0 = time.perf_counter()
    for _ in range(reps):
        for n in ("q", "k"):
            oracle.rmsnorm(d[n], d["gamma_" + n], w.eps, threads=1)
    cpu_ms = (time.perf_counter() - t0) / reps * 1e3
    ops.bench_fused(q, k, gq, gk, w.n_shards, w.eps, oq, ok, 200)
    r = 2000
    us = timed(lambda _: ops.bench_fused(q, k, gq, gk, w.n_shards, w.eps, oq, ok, r),
               1, stream, torch) * 1e3 / r
    return {"workload": "T=8, Q and K width 256, fp32, 2 logical shards",
            "cpu_oracle_ms_per_call": round(cpu_ms, 4), "cpu_oracle_threads": 1,
            "device_us_per_call": round(us, 2)}


def cpu_baseline(w, d, budget_s=10.0):
    """The fp64 oracle on the workload's rows, sized to about budget_s of CPU time.

    Rows are taken from the front of the batch; when one pass over every row takes less
    than the budget, whole passes are repeated until it is spent."""
    from oracle import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    probe = min(w.T, 256)
    t0 = time.perf_counter()
    for n in ("q", "k"):
        oracle.rmsnorm(d[n][:probe], d["gamma_" + n], w.eps, threads=threads)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(max(probe, min(w.T, budget_s / max(per_row, 1e-9))))
    passes, sec = 0, 0.0
    t0 = time.perf_counter()
    while True:
        for n in ("q", "k"):
            oracle.rmsnorm(d[n][:rows], d["gamma_" + n], w.eps, threads=threads)
        passes += 1
        sec = time.perf_counter() - t0
        if sec >= 0.8 * budget_s or rows < w.T:
            break
    nbytes = w.with_T(rows).algorithmic_bytes() * passes
    what = f"all {w.T} tokens" if rows == w.T else f"first {rows} of {w.T} tokens"
    return {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{passes} pass(es) over {what} of the prefill workload (Q and K, fp64 C "
                      f"loops, rows split over {threads} threads), {sec:.2f} s"}


def cpu_host(w, d, budget_s=2.5):
    """The host the baseline ran on: CPU model, usable cores, and the oracle's rate on
    one core (rows from the front of the prefill batch for about budget_s)."""
    from oracle import oracle
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rows, sec = 64, 0.0
    while True:
        t0 = time.perf_counter()
        for n in ("q", "k"):
            oracle.rmsnorm(d[n][:rows], d["gamma_" + n], w.eps, threads=1)
        sec = time.perf_counter() - t0
        if sec >= 0.25 * budget_s or rows >= w.T:
            break
        rows = min(w.T, rows * 4)
    return {"model": model, "os_cpu_count": os.cpu_count(),
            "single_core_GBs": round(w.with_T(rows).algorithmic_bytes() / sec / 1e9, 4),
            "single_core_sample": f"first {rows} of {w.T} tokens, Q and K, {sec:.2f} s"}


_DRAW_FIELDS = ("T", "Hq", "Hk", "dtype", "dist", "sigma", "outlier_frac", "outlier_scale",
                "mu", "seed")


def host_inputs(w, cache):
    """make_host(w), reusing the activations of an earlier workload in ``cache`` whose
    draws are the same (same streams, distribution, shape and storage format): then
    only the parameters are drawn, from a one-token draw (their streams are separate,
    so they equal the full draw's)."""
    from layerwise_qk_norm_amd import inputs
    key = tuple(getattr(w, f) for f in _DRAW_FIELDS)
    if key in cache:
        d = inputs.make_host(w.with_T(1))
        d["q"], d["k"] = cache[key]
        return d
    d = inputs.make_host(w)
    cache[key] = (d["q"], d["k"])
    return d


def prepare_all(torch, pmc: bool):
    """Every leg's inputs drawn on the host and copied to the device, before any
    timing. Returns {leg name: prepared tensors} and the host prefill arrays."""
    from layerwise_qk_norm_amd import inputs
    dev = "cuda:0"
    prep, cache = {}, {}
    w = inputs.PREFILL
    d = host_inputs(w, cache)
    prep["prefill"] = (w,) + upload_sets(w, d, torch, 1 if pmc else 2)
    w8 = inputs.PREFILL_E4M3
    d8 = inputs.make_host(w8)
    sets8 = 1 if pmc else 3
    prep["prefill_to_bf16"] = (w8,) + upload_sets(w8, d8, torch, sets8)
    w88 = dataclasses.replace(w8, out_dtype="e4m3")
    prep["prefill_to_e4m3"] = (w88,) + upload_sets(w88, d8, torch, sets8)
    del d8
    wl = inputs.LN_PREFILL
    dl = host_inputs(wl, cache)
    par = {n: inputs.to_device(dl[n], dev, torch) for n in ("gamma_q", "gamma_k", "beta_q", "beta_k")}
    lb = []
    for _ in range(1 if pmc else 2):
        q, k = inputs.to_device(dl["q"], dev, torch), inputs.to_device(dl["k"], dev, torch)
        lb.append((q, k, torch.empty_like(q), torch.empty_like(k)))
    prep["ln_prefill"] = (wl, par, lb)
    del dl
    wh = inputs.HW_PREFILL
    dh = host_inputs(wh, cache)
    prep["headwise"] = (wh,) + upload_sets(wh, dh, torch, 1 if pmc else 2)
    del dh
    wg = inputs.GQA
    dg = inputs.make_host(wg)
    prep["gqa"] = (wg,) + upload_sets(wg, dg, torch, 1 if pmc else 3)
    del dg
    if not pmc:
        wd = inputs.DECODE
        dd = inputs.make_host(wd)
        gq, gk, b = upload_sets(wd, dd, torch, 1)
        prep["decode"] = (wd, gq, gk, b[0])
        wld = inputs.LN_DECODE
        dld = inputs.make_host(wld)
        t = {n: inputs.to_device(dld[n], dev, torch) for n in dld}
        prep["ln_decode"] = (wld, t, (torch.empty_like(t["q"]), torch.empty_like(t["k"])))
        wde = inputs.DECODE_E4M3
        dde = inputs.make_host(wde)
        gq, gk, b = upload_sets(wde, dde, torch, 1)
        prep["decode_e4m3"] = (wde, gq, gk, b[0])
        wt = inputs.TINY
        dt = inputs.make_host(wt)
        gq, gk, b = upload_sets(wt, dt, torch, 1)
        q, k, oq, ok = b[0]
        prep["tiny"] = (wt, dt, (q, k, gq, gk, oq, ok))
    torch.cuda.synchronize()
    return prep, d


def run_pmc(torch, prep, plans_path=""):
    """Five launches of each kernel whose counters are collected, plus the copy of
    known size (the prefill workload's Q and K)."""
    from layerwise_qk_norm_amd import ops
    w, gq, gk, bufs = prep["prefill"]
    q, k, oq, ok = bufs[0]
    for _ in range(5):
        ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=oq, out_k=ok)
        ops.bench_copy(q, k, oq, ok)
    for key in ("prefill_to_bf16", "prefill_to_e4m3", "gqa"):
        w8, g8q, g8k, b8 = prep[key]
        q, k, oq, ok = b8[0]
        for _ in range(5):
            ops.layerwise_fwd(q, k, g8q, g8k, w8.n_shards, w8.eps, out_q=oq, out_k=ok)
    wl, par, lb = prep["ln_prefill"]
    q, k, oq, ok = lb[0]
    for _ in range(5):
        ops.layernorm_fwd(q, k, par["gamma_q"], par["gamma_k"], wl.n_shards, wl.eps,
                          beta_q=par["beta_q"], beta_k=par["beta_k"], out_q=oq, out_k=ok)
    wh, hq, hk, hb = prep["headwise"]
    q, k, oq, ok = hb[0]
    for _ in range(5):
        ops.headwise_fwd(q, k, hq, hk, wh.head_dim, wh.eps, out_q=oq, out_k=ok)
    torch.cuda.synchronize()
    assert ops.check_fault() == ops.QKN_OK
    # the launch plan of each profiled kernel, for the traffic summaries
    plans = {"prefill": ops.current_plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards),
             "headwise": HEADWISE_PLAN}
    for key in ("prefill_to_bf16", "prefill_to_e4m3", "gqa"):
        wk = prep[key][0]
        plans[key] = ops.current_plan(wk.fmt, wk.T, wk.Hq, wk.Hk, wk.n_shards)
    plans["ln_prefill"] = ops.current_plan(wl.fmt, wl.T, wl.Hq, wl.Hk, wl.n_shards)
    if plans_path:
        os.makedirs(os.path.dirname(os.path.abspath(plans_path)), exist_ok=True)
        json.dump(plans, open(plans_path, "w"), indent=1, sort_keys=True)
    log("pmc mode done: 5 launches each of the fused bf16 prefill kernel and of the copy of "
        f"{w.T * (w.Hq + w.Hk) * w.elem_bytes} bytes read, then 5 each of fused E4M3->bf16 and "
        "E4M3->E4M3 prefill, GQA, LayerNorm prefill and headwise prefill")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc", action="store_true", help="counter-collection mode")
    ap.add_argument("--pmc-plans", default="", help="counter-collection mode: write each leg's "
                    "launch plan to this JSON file (the traffic summaries key on it)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on one GPU; --gpus N with N > 1 is not supported "
              "(the shards are logical shards on one device)", file=sys.stderr)
        sys.exit(2)

    import torch
    from layerwise_qk_norm_amd import ops
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    ops.lib()  # raises if the HIP library is missing
    stream = torch.cuda.current_stream()

    log("drawing and uploading every leg's inputs ...")
    t0 = time.perf_counter()
    prep, d = prepare_all(torch, args.pmc)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    if args.pmc:
        run_pmc(torch, prep, args.pmc_plans)
        return

    w, gq, gk, bufs = prep["prefill"]
    nbytes = w.algorithmic_bytes()
    plan = ops.current_plan(w.dtype, w.T, w.Hq, w.Hk, w.n_shards)
    log(f"plan: {plan}")

    def fused(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=oq, out_k=ok)

    def copy(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.bench_copy(q, k, oq, ok)

    leg = Leg(fused, stream, torch)
    pre = leg.run_preroll()
    log(f"preroll: {pre}")
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("fused kernel reported an exchange timeout during the preroll")
    log(f"timing {args.steps} fused steps after {args.warmup} warmup steps ...")
    ms = leg.measure(args.warmup, args.steps)
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("fused kernel reported an exchange timeout")
    gbs = nbytes / (ms * 1e-3) / 1e9

    log("timing copy ceiling, the launch skeleton and the split path ...")
    copy_bytes = nbytes - (w.Hq + w.Hk) * w.elem_bytes
    copy_ms, copy_pre = timed_leg(copy, args, stream, torch)
    copy_gbs = copy_bytes / (copy_ms * 1e-3) / 1e9
    prep["copy_bytes"], prep["copy_ms"] = copy_bytes, copy_ms
    skel = skeleton(args, stream, torch, bufs, w, w.fmt, copy_bytes, ms)
    ops.set_option("force_split", 1)
    try:
        split_ms, split_pre = timed_leg(fused, args, stream, torch)
    finally:
        ops.set_option("force_split", 0)

    # decode: device time per call (events around each call) and host-visible time
    log("timing decode ...")
    wd, dgq, dgk, (q, k, oq, ok) = prep["decode"]

    def dec(_):
        ops.layerwise_fwd(q, k, dgq, dgk, wd.n_shards, wd.eps, out_q=oq, out_k=ok)

    for i in range(50):
        dec(i)
    torch.cuda.synchronize()
    per_call = []
    for i in range(200):
        per_call.append(timed(dec, 1, stream, torch))
    n_host = 1000
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_host):
        dec(i)
    torch.cuda.synchronize()
    host_us = (time.perf_counter() - t0) / n_host * 1e6
    dev_us_b2b = timed(dec, n_host, stream, torch) * 1e3
    # the same calls through a prepared call (validated once), as a decode loop
    # that reuses its tensors would issue them
    pcall = ops.prepare_layerwise_fwd(q, k, dgq, dgk, wd.n_shards, wd.eps, out_q=oq, out_k=ok)
    for i in range(50):
        pcall()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_host):
        pcall()
    torch.cuda.synchronize()
    host_prep_us = (time.perf_counter() - t0) / n_host * 1e6
    # device rate without host-language overhead: launches issued from C
    reps = 2000
    ops.bench_fused(q, k, dgq, dgk, wd.n_shards, wd.eps, oq, ok, 200)
    c_us = timed(lambda _: ops.bench_fused(q, k, dgq, dgk, wd.n_shards, wd.eps, oq, ok, reps),
                 1, stream, torch) * 1e3 / reps
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("decode reported an exchange timeout")

    log("timing E4M3 activations ...")
    e4m3 = leg_e4m3(args, torch, stream, prep)
    log("timing LayerNorm ...")
    layernorm = leg_layernorm(args, torch, stream, prep)
    log("timing headwise ...")
    headwise = leg_headwise(args, torch, stream, prep)
    log("timing the GQA workload ...")
    gqa = leg_gqa(args, torch, stream, prep)
    log("timing the tiny workload ...")
    tiny = leg_tiny(torch, stream, prep)

    traffic = read_traffic(TRAFFIC_SUMMARY, plan)
    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, 2^2) activations, U(0.5, 1.5) gamma)",
        "config": {"workload": "prefill: T=16384, Q and K width 5120, bf16, 2 logical shards",
                   "T": w.T, "Hq": w.Hq, "Hk": w.Hk, "n_shards": w.n_shards, "eps": w.eps,
                   "algorithmic_bytes": nbytes, "plan": plan},
        "preroll": pre,
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "decode": {"workload": "T=64, Q and K width 4096, bf16, 4 logical shards",
                   "device_us_per_call": round(c_us, 2),
                   "event_us_single_call_median": round(float(np.median(per_call)) * 1e3, 2),
                   "python_back_to_back_us_per_call": round(dev_us_b2b, 2),
                   "host_visible_us_per_call": round(host_us, 2),
                   "host_visible_prepared_us_per_call": round(host_prep_us, 2)},
        "copy": {"GBs": round(copy_gbs, 1), "ms": round(copy_ms, 5),
                 "fused_frac_of_copy": round(gbs / copy_gbs, 4), "preroll": copy_pre},
        "skeleton": skel,
        "split": {"GBs": round(nbytes / (split_ms * 1e-3) / 1e9, 1), "ms": round(split_ms, 5),
                  "preroll": split_pre},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "e4m3": e4m3,
        "layernorm": layernorm,
        "headwise": headwise,
        "gqa": gqa,
        "tiny": tiny,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(w, d)
        out["cpu_host"] = cpu_host(w, d)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
