#!/usr/bin/env python3
"""Benchmark of the fused Q+K layerwise RMSNorm on one MI355X.

One step = one fused call (every stage of the path: shard partials, scalar
exchange and combine, x*gamma, final scaling) over the prefill workload:
T=16384 tokens, Q and K width 5120, bf16, 2 logical shards, inputs resident
in HBM. Prints ONE JSON line on stdout; progress goes to stderr.

Besides the headline (GB/s of algorithmic bytes), the line carries:
  decode      -- the T=64 decode workload: device and host-visible us per call
  copy        -- a plain copy of the same bytes (achievable-bandwidth ceiling)
  split       -- the three-kernel split path on the same workload
  roofline    -- the fused kernel against MI355X peak HBM bandwidth
  cpu_baseline-- the fp64 oracle timed on this host's cores on a sample
  cpu_host    -- the host CPU model and the oracle's rate on one core

  e4m3        -- FP8-E4M3 activations (bf16 gamma) on the prefill shape with bf16
                 and with E4M3 outputs, each against the HBM roofline, and the
                 decode shape in us per call
  layernorm   -- LayerNorm (two additive shard statistics, gamma and beta) on the
                 prefill shape against the HBM roofline, and the decode shape
  headwise    -- headwise QK-Norm (one factor per head of 128 columns) on the
                 prefill shape against the HBM roofline
  gqa         -- the GQA-shaped workload (Q width 5120, K width 1024, 4 shards)
                 against the HBM roofline

Modes: ``--pmc`` runs only the kernels whose counters are collected
(fused prefill in bf16, in E4M3->bf16, in E4M3->E4M3 and as LayerNorm, headwise
prefill, and the copy of known size), for rocprofv3 --pmc runs.
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
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fused_prefill_T16384_traffic.txt")
TRAFFIC_SUMMARY_E4M3 = os.path.join(ROOT, "profiles", "fused_prefill_e4m3_T16384_traffic.txt")
TRAFFIC_SUMMARY_LN = os.path.join(ROOT, "profiles", "fused_layernorm_prefill_T16384_traffic.txt")
TRAFFIC_SUMMARY_E4M3_E4M3 = os.path.join(ROOT, "profiles", "fused_prefill_e4m3_to_e4m3_T16384_traffic.txt")
TRAFFIC_SUMMARY_HW = os.path.join(ROOT, "profiles", "headwise_prefill_T16384_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def read_traffic(path=TRAFFIC_SUMMARY):
    """HBM bytes per launch from a committed counter summary, if it is current."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    from layerwise_qk_norm_amd.profiling import kernel_source_sha
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed(fn, steps, stream, torch):
    """Average ms per call of ``fn`` over ``steps`` back-to-back calls (HIP events)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def device_workload(w, torch, sets=1):
    from layerwise_qk_norm_amd import inputs
    d = inputs.make_host(w)
    dev = "cuda:0"
    gq, gk = inputs.to_device(d["gamma_q"], dev, torch), inputs.to_device(d["gamma_k"], dev, torch)
    odt = {"bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.float8_e4m3fn}[w.out]
    bufs = []
    for s in range(sets):
        q = inputs.to_device(d["q"], dev, torch)
        k = inputs.to_device(d["k"], dev, torch)
        bufs.append((q, k, torch.empty(q.shape, dtype=odt, device=dev),
                     torch.empty(k.shape, dtype=odt, device=dev)))
    return d, gq, gk, bufs


def roofline(nbytes, ms, traffic):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}


def bench_layernorm(args, torch, stream, timed):
    """LayerNorm with two additive shard statistics on the prefill and decode shapes."""
    from layerwise_qk_norm_amd import inputs, ops
    out = {}
    w = inputs.LN_PREFILL
    d = inputs.make_host(w)
    dev = "cuda:0"
    par = {n: inputs.to_device(d[n], dev, torch) for n in ("gamma_q", "gamma_k", "beta_q", "beta_k")}
    bufs = []
    for _ in range(2):
        q, k = inputs.to_device(d["q"], dev, torch), inputs.to_device(d["k"], dev, torch)
        bufs.append((q, k, torch.empty_like(q), torch.empty_like(k)))

    def fused(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.layernorm_fwd(q, k, par["gamma_q"], par["gamma_k"], w.n_shards, w.eps,
                          beta_q=par["beta_q"], beta_k=par["beta_k"], out_q=oq, out_k=ok)

    for i in range(args.warmup):
        fused(i)
    ms = timed(fused, args.steps, stream, torch)
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("LayerNorm prefill reported an exchange timeout")
    nbytes = w.algorithmic_bytes()
    out["prefill"] = {
        "workload": f"T={w.T}, Q and K width {w.Hq}, bf16, gamma and beta, {w.n_shards} logical shards",
        "algorithmic_bytes": nbytes, "ms": round(ms, 5),
        "plan": ops.current_plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards),
        "roofline": roofline(nbytes, ms, read_traffic(TRAFFIC_SUMMARY_LN))}
    del bufs
    torch.cuda.empty_cache()
    wd = inputs.LN_DECODE
    dd = inputs.make_host(wd)
    t = {n: inputs.to_device(dd[n], dev, torch) for n in dd}
    oq, ok = torch.empty_like(t["q"]), torch.empty_like(t["k"])

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


def bench_gqa(args, torch, stream, timed):
    """The GQA-shaped workload (T=8192, Q width 5120, K width 1024, 4 logical shards).
    One call moves 201 MB, less than the 256 MB Infinity Cache, so three buffer sets
    rotate (604 MB) and every call streams from HBM."""
    from layerwise_qk_norm_amd import inputs, ops
    w = inputs.GQA
    _, gq, gk, bufs = device_workload(w, torch, sets=3)

    def fused(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=oq, out_k=ok)

    for i in range(args.warmup):
        fused(i)
    ms = timed(fused, args.steps, stream, torch)
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("GQA workload reported an exchange timeout")
    nbytes = w.algorithmic_bytes()
    out = {"workload": f"T={w.T}, Q width {w.Hq}, K width {w.Hk}, bf16, {w.n_shards} logical shards",
           "algorithmic_bytes": nbytes, "ms": round(ms, 5),
           "plan": ops.current_plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards),
           "roofline": roofline(nbytes, ms, None)}
    del bufs
    torch.cuda.empty_cache()
    return out


def bench_headwise(args, torch, stream, timed):
    """Headwise QK-Norm (one factor per head of 128 columns) on the prefill shape."""
    from layerwise_qk_norm_amd import inputs, ops
    w = inputs.HW_PREFILL
    d = inputs.make_host(w)
    dev = "cuda:0"
    gq, gk = inputs.to_device(d["gamma_q"], dev, torch), inputs.to_device(d["gamma_k"], dev, torch)
    bufs = []
    for _ in range(2):
        q, k = inputs.to_device(d["q"], dev, torch), inputs.to_device(d["k"], dev, torch)
        bufs.append((q, k, torch.empty_like(q), torch.empty_like(k)))

    def fused(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.headwise_fwd(q, k, gq, gk, w.head_dim, w.eps, out_q=oq, out_k=ok)

    for i in range(args.warmup):
        fused(i)
    ms = timed(fused, args.steps, stream, torch)
    nbytes = w.algorithmic_bytes()
    out = {"prefill": {
        "workload": f"T={w.T}, Q and K width {w.Hq} ({w.Hq // w.head_dim} heads of {w.head_dim}), bf16",
        "algorithmic_bytes": nbytes, "ms": round(ms, 5),
        "roofline": roofline(nbytes, ms, read_traffic(TRAFFIC_SUMMARY_HW))}}
    del bufs
    torch.cuda.empty_cache()
    return out


def bench_e4m3(args, torch, stream, timed):
    """FP8-E4M3 activations: prefill with bf16 and with E4M3 outputs, decode."""
    from layerwise_qk_norm_amd import inputs, ops
    out = {}
    for w in (inputs.PREFILL_E4M3, dataclasses.replace(inputs.PREFILL_E4M3, out_dtype="e4m3")):
        _, gq, gk, bufs = device_workload(w, torch, sets=2)

        def fused(i):
            q, k, oq, ok = bufs[i % len(bufs)]
            ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=oq, out_k=ok)

        for i in range(args.warmup):
            fused(i)
        ms = timed(fused, args.steps, stream, torch)
        if ops.check_fault() != ops.QKN_OK:
            raise RuntimeError("E4M3 prefill reported an exchange timeout")
        nbytes = w.algorithmic_bytes()
        traffic = read_traffic(TRAFFIC_SUMMARY_E4M3 if w.out == "bf16" else TRAFFIC_SUMMARY_E4M3_E4M3)
        out[f"prefill_to_{w.out}"] = {
            "workload": f"T={w.T}, Q and K width {w.Hq}, E4M3 in, bf16 gamma, {w.out} out, "
                        f"{w.n_shards} logical shards",
            "algorithmic_bytes": nbytes, "ms": round(ms, 5),
            "plan": ops.current_plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards),
            "roofline": roofline(nbytes, ms, traffic)}
        del bufs
        torch.cuda.empty_cache()
    wd = inputs.DECODE_E4M3
    _, dgq, dgk, dbufs = device_workload(wd, torch, sets=1)
    q, k, oq, ok = dbufs[0]
    ops.bench_fused(q, k, dgq, dgk, wd.n_shards, wd.eps, oq, ok, 200)
    reps = 2000
    c_us = timed(lambda _: ops.bench_fused(q, k, dgq, dgk, wd.n_shards, wd.eps, oq, ok, reps),
                 1, stream, torch) * 1e3 / reps
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("E4M3 decode reported an exchange timeout")
    out["decode"] = {"workload": "T=64, Q and K width 4096, E4M3 in and out, 4 logical shards",
                     "device_us_per_call": round(c_us, 2)}
    return out


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


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc", action="store_true", help="counter-collection mode")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on one GPU; --gpus N with N > 1 is not supported "
              "(the shards are logical shards on one device)", file=sys.stderr)
        sys.exit(2)

    import torch
    from layerwise_qk_norm_amd import inputs, ops
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    ops.lib()  # raises if the HIP library is missing
    stream = torch.cuda.current_stream()

    w = inputs.PREFILL
    nbytes = w.algorithmic_bytes()
    log(f"generating {w.name} inputs ...")
    d, gq, gk, bufs = device_workload(w, torch, sets=1 if args.pmc else 2)
    plan = ops.current_plan(w.dtype, w.T, w.Hq, w.Hk, w.n_shards)
    log(f"plan: {plan}")

    def fused(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=oq, out_k=ok)

    def copy(i):
        q, k, oq, ok = bufs[i % len(bufs)]
        ops.bench_copy(q, k, oq, ok)

    if args.pmc:
        for i in range(5):
            fused(i)
            copy(i)
        for w8 in (inputs.PREFILL_E4M3, dataclasses.replace(inputs.PREFILL_E4M3, out_dtype="e4m3")):
            _, gq8, gk8, b8 = device_workload(w8, torch, sets=1)
            for i in range(5):
                q, k, oq, ok = b8[0]
                ops.layerwise_fwd(q, k, gq8, gk8, w8.n_shards, w8.eps, out_q=oq, out_k=ok)
            del b8
        wl = inputs.LN_PREFILL
        dl = inputs.make_host(wl)
        tl = {n: inputs.to_device(dl[n], "cuda:0", torch) for n in dl}
        for i in range(5):
            ops.layernorm_fwd(tl["q"], tl["k"], tl["gamma_q"], tl["gamma_k"], wl.n_shards, wl.eps,
                              beta_q=tl["beta_q"], beta_k=tl["beta_k"])
        del tl
        wh = inputs.HW_PREFILL
        dh = inputs.make_host(wh)
        th = {n: inputs.to_device(dh[n], "cuda:0", torch) for n in ("q", "k", "gamma_q", "gamma_k")}
        for i in range(5):
            ops.headwise_fwd(th["q"], th["k"], th["gamma_q"], th["gamma_k"], wh.head_dim, wh.eps)
        torch.cuda.synchronize()
        assert ops.check_fault() == ops.QKN_OK
        log("pmc mode done: 5 fused bf16 prefill launches, 5 copy launches of "
            f"{w.T * (w.Hq + w.Hk) * w.elem_bytes} bytes read, 5 fused E4M3->bf16 and 5 E4M3->E4M3 "
            "prefill launches, 5 fused LayerNorm prefill launches, 5 headwise prefill launches")
        return

    for i in range(args.warmup):
        fused(i)
    torch.cuda.synchronize()
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("fused kernel reported an exchange timeout during warmup")
    log(f"timing {args.steps} fused steps ...")
    ms = timed(fused, args.steps, stream, torch)
    if ops.check_fault() != ops.QKN_OK:
        raise RuntimeError("fused kernel reported an exchange timeout")
    gbs = nbytes / (ms * 1e-3) / 1e9

    log("timing copy ceiling and split path ...")
    for i in range(3):
        copy(i)
    copy_ms = timed(copy, args.steps, stream, torch)
    copy_gbs = (nbytes - (w.Hq + w.Hk) * w.elem_bytes) / (copy_ms * 1e-3) / 1e9
    ops.set_option("force_split", 1)
    for i in range(3):
        fused(i)
    split_ms = timed(fused, args.steps, stream, torch)
    ops.set_option("force_split", 0)

    # decode: device time per call (events around each call) and host-visible time
    log("timing decode ...")
    wd = inputs.DECODE
    dd, dgq, dgk, dbufs = device_workload(wd, torch, sets=1)
    q, k, oq, ok = dbufs[0]

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
    e4m3 = bench_e4m3(args, torch, stream, timed)
    log("timing LayerNorm ...")
    layernorm = bench_layernorm(args, torch, stream, timed)
    log("timing headwise ...")
    headwise = bench_headwise(args, torch, stream, timed)
    log("timing the GQA workload ...")
    gqa = bench_gqa(args, torch, stream, timed)

    traffic = read_traffic()
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
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "decode": {"workload": "T=64, Q and K width 4096, bf16, 4 logical shards",
                   "device_us_per_call": round(c_us, 2),
                   "event_us_single_call_median": round(float(np.median(per_call)) * 1e3, 2),
                   "python_back_to_back_us_per_call": round(dev_us_b2b, 2),
                   "host_visible_us_per_call": round(host_us, 2),
                   "host_visible_prepared_us_per_call": round(host_prep_us, 2)},
        "copy": {"GBs": round(copy_gbs, 1), "ms": round(copy_ms, 5),
                 "fused_frac_of_copy": round(gbs / copy_gbs, 4)},
        "split": {"GBs": round(nbytes / (split_ms * 1e-3) / 1e9, 1), "ms": round(split_ms, 5)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "e4m3": e4m3,
        "layernorm": layernorm,
        "headwise": headwise,
        "gqa": gqa,
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
