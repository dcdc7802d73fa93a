"""Summaries of rocprofv3 output for the committed ``profiles/`` directory.

``python -m layerwise_qk_norm_amd.profiling trace STATS_CSV OUT_TXT --cmd "..."
  [--kernel-trace TRACE_CSV --window KERNEL:START:COUNT]`` writes the per-kernel duration
  table of a ``--kernel-trace --stats`` run and, with a window, the average over one
  run of consecutive dispatches (the benchmark's timed steps, after its warmup).
  ``--bench-json LINE_JSON --leg PATH --kernel NAME`` takes the window from the
  profiled benchmark's own JSON line instead: the leg's timed steps start after its
  preroll calls and the warmup (``--leg`` is the dotted key of the leg, e.g. ``gqa``
  or ``e4m3.prefill_to_bf16``; empty for the headline leg).
``python -m layerwise_qk_norm_amd.profiling sq OUT_TXT CSV... --cmd "..."`` writes the
  instruction-issue counters (SQ_*) of the fused prefill kernel next to the copy
  kernel's, averaged per dispatch, from one or more ``--pmc`` runs.
``python -m layerwise_qk_norm_amd.profiling traffic FETCH_CSV WRITE_CSV OUT_TXT --cmd-fetch
  "..." --cmd-write "..."`` writes HBM bytes per launch of the fused prefill kernel
  from two ``--pmc`` runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch). Each counter
  is scaled by what it reads for the copy kernel of known size in the same run
  (the copy reads and writes exactly the prefill workload's Q and K bytes).

Summaries record the hash of the device code they measured (the kernels'
header) and, for traffic, the launch plan of the kernel (from the plans file that
``bench.py --pmc`` writes); the benchmark uses a traffic figure only while both
match the current sources and the plan it launches.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
# the device code: every kernel and its inlined helpers live in this header
KERNEL_SOURCES = [os.path.join(PKG, "csrc", "qknorm_kernels.hpp")]

# The copy kernel of the --pmc run moves the prefill workload's Q and K:
# 16384 x (5120 + 5120) bf16 values read and the same written.
COPY_BYTES = 16384 * (5120 + 5120) * 2


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def short(name: str) -> str:
    return name.replace("(qkn::FusedParams)", "").replace("void ", "")[:110]


def window_stats(trace_csv: str, kernel: str, start: int, count: int):
    """Durations of dispatches [start, start+count) of the kernel whose name contains
    ``kernel``, from a ``--kernel-trace`` CSV (dispatch order = launch order)."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    sel = rows[start:start + count]
    if len(sel) < count:
        raise ValueError(f"only {len(rows)} dispatches of {kernel!r}")
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
    st = [int(r["Start_Timestamp"]) for r in sel]
    gap = [(st[i + 1] - st[i]) / 1e3 for i in range(len(st) - 1)]
    return {"name": sel[0]["Kernel_Name"], "n": len(dur), "avg_us": statistics.mean(dur),
            "min_us": min(dur), "max_us": max(dur),
            "start_to_start_us": statistics.mean(gap) if gap else float("nan")}


def bench_window(line_json: str, leg: str, kernel: str) -> str:
    """KERNEL:START:COUNT of a leg's timed steps in a profiled benchmark run: the
    leg's kernel was launched ``preroll.calls`` times, then ``warmup`` times, then
    ``steps`` timed times (each leg's kernel is launched by that leg only)."""
    import json
    d = json.load(open(line_json))
    node = d
    for part in [p for p in leg.split(".") if p]:
        node = node[part]
    start = int(node["preroll"]["calls"]) + int(d["warmup"])
    return f"{kernel}:{start}:{int(d['steps'])}"


def summarize_trace(stats_csv: str, out_txt: str, cmd: str, note: str = "",
                    trace_csv: str = "", window: str = ""):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {cmd}",
             f"kernel_source_sha: {kernel_source_sha()}"]
    if note:
        lines.append(f"# {note}")
    lines.append(f"{'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
    for r in rows:
        lines.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.3f} "
                     f"{float(r['MinNs']) / 1e3:10.3f} {float(r['MaxNs']) / 1e3:10.3f} "
                     f"{float(r['Percentage']):6.2f}  {short(r['Name'])}")
    if trace_csv and window:
        kernel, start, count = window.rsplit(":", 2)
        w = window_stats(trace_csv, kernel, int(start), int(count))
        lines += [f"# timed window: dispatches {start}..{int(start) + int(count) - 1} of "
                  f"{short(w['name'])}",
                  f"window_dispatches: {w['n']}",
                  f"window_avg_us: {w['avg_us']:.3f}",
                  f"window_min_us: {w['min_us']:.3f}",
                  f"window_max_us: {w['max_us']:.3f}",
                  f"window_start_to_start_us: {w['start_to_start_us']:.3f}"]
    open(out_txt, "w").write("\n".join(lines) + "\n")


def _per_kernel(csv_path: str):
    out = {}
    for r in csv.DictReader(open(csv_path)):
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def plan_line(plan) -> str:
    """The launch plan as the one-line JSON the summaries and the benchmark compare."""
    import json
    return json.dumps(plan, sort_keys=True)


def summarize_traffic(fetch_csv: str, write_csv: str, out_txt: str, cmd_fetch: str,
                      cmd_write: str, algorithmic_bytes: int, kernel: str = "fused_qknorm_kernel<qkn::Bf16",
                      title: str = "fused prefill kernel (T=16384, Q and K width 5120, bf16, N=2)",
                      plan=None):
    fetch, write = _per_kernel(fetch_csv), _per_kernel(write_csv)
    copy_name = next(n for n in fetch if "copy_ceiling_kernel" in n)
    fused_name = next(n for n in fetch if kernel in n)
    kib_copy_f = statistics.mean(fetch[copy_name])
    kib_copy_w = statistics.mean(write[copy_name])
    scale_f = (COPY_BYTES / 1024) / kib_copy_f
    scale_w = (COPY_BYTES / 1024) / kib_copy_w
    kib_f = statistics.mean(fetch[fused_name])
    kib_w = statistics.mean(write[fused_name])
    fetched = kib_f * scale_f * 1024
    written = kib_w * scale_w * 1024
    traffic = fetched + written
    lines = [
        f"# HBM traffic of the {title}",
        f"# command (FETCH_SIZE): {cmd_fetch}",
        f"# command (WRITE_SIZE): {cmd_write}",
        f"# copy kernel of known size: {COPY_BYTES} B read and {COPY_BYTES} B written",
        f"kernel_source_sha: {kernel_source_sha()}",
        f"kernel: {short(fused_name)}",
        f"plan: {plan_line(plan) if plan is not None else 'none'}",
        f"dispatches: {len(fetch[fused_name])} (FETCH_SIZE), {len(write[fused_name])} (WRITE_SIZE)",
        f"fetch_kib_per_dispatch: {kib_f:.3f}",
        f"write_kib_per_dispatch: {kib_w:.3f}",
        f"copy_fetch_kib_per_dispatch: {kib_copy_f:.3f}",
        f"copy_write_kib_per_dispatch: {kib_copy_w:.3f}",
        f"copy_scale_fetch: {scale_f:.5f}",
        f"copy_scale_write: {scale_w:.5f}",
        f"fetched_bytes_per_launch: {fetched:.0f}",
        f"written_bytes_per_launch: {written:.0f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"algorithmic_bytes_per_launch: {algorithmic_bytes}",
        f"traffic_over_algorithmic: {traffic / algorithmic_bytes:.4f}",
    ]
    open(out_txt, "w").write("\n".join(lines) + "\n")


def _counters(csv_path: str):
    """{kernel: {counter: [value per dispatch]}} of one --pmc run."""
    out = {}
    for r in csv.DictReader(open(csv_path)):
        out.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    return out


def summarize_sq(csvs, out_txt: str, cmds, kernel: str, title: str):
    """Instruction-issue counters (per dispatch, averaged) of one kernel and of the
    copy kernel of the same run, from one or more --pmc runs."""
    fused, copy = {}, {}
    for path in csvs:
        per = _counters(path)
        fname = next(n for n in per if kernel in n)
        cname = next(n for n in per if "copy_ceiling_kernel" in n)
        for c, v in per[fname].items():
            fused[c] = statistics.mean(v)
        for c, v in per[cname].items():
            copy[c] = statistics.mean(v)
    lines = [f"# SQ instruction counters of the {title}, averaged per dispatch"]
    lines += [f"# command: {c}" for c in cmds]
    lines += [f"kernel_source_sha: {kernel_source_sha()}", f"kernel: {short(fname)}",
              f"{'counter':24s} {'fused':>16s} {'copy':>16s}"]
    for c in sorted(fused):
        lines.append(f"{c:24s} {fused[c]:16.0f} {copy.get(c, float('nan')):16.0f}")
    waves = fused.get("SQ_WAVES")
    if waves and "SQ_INSTS_VALU" in fused:
        lines.append(f"valu_insts_per_wave: {fused['SQ_INSTS_VALU'] / waves:.0f}")
    if "SQ_ACTIVE_INST_VALU" in fused and "SQ_WAVE_CYCLES" in fused:
        lines.append("valu_active_over_wave_cycles: "
                     f"{fused['SQ_ACTIVE_INST_VALU'] / fused['SQ_WAVE_CYCLES']:.3f}")
    if "SQ_WAIT_INST_ANY" in fused and "SQ_WAVE_CYCLES" in fused:
        lines.append("wait_inst_any_over_wave_cycles: "
                     f"{fused['SQ_WAIT_INST_ANY'] / fused['SQ_WAVE_CYCLES']:.3f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out_txt")
    t.add_argument("--cmd", required=True)
    t.add_argument("--note", default="")
    t.add_argument("--kernel-trace", default="", help="kernel trace CSV for --window")
    t.add_argument("--window", default="",
                   help="KERNEL_SUBSTRING:START:COUNT, dispatches averaged on their own")
    t.add_argument("--bench-json", default="", help="the profiled run's JSON line")
    t.add_argument("--leg", default="", help="dotted key of the leg in that line")
    t.add_argument("--kernel", default="", help="kernel-name substring of the leg's kernel")
    f = sub.add_parser("traffic")
    f.add_argument("fetch_csv")
    f.add_argument("write_csv")
    f.add_argument("out_txt")
    f.add_argument("--cmd-fetch", required=True)
    f.add_argument("--cmd-write", required=True)
    f.add_argument("--algorithmic-bytes", type=int, default=671_109_120)
    f.add_argument("--kernel", default="fused_qknorm_kernel<qkn::Bf16",
                   help="substring of the kernel name to summarise")
    f.add_argument("--title", default="fused prefill kernel (T=16384, Q and K width 5120, bf16, N=2)")
    f.add_argument("--plans", default="", help="plans file written by bench.py --pmc")
    f.add_argument("--leg", default="", help="key of the kernel's launch in the plans file")
    q = sub.add_parser("sq")
    q.add_argument("out_txt")
    q.add_argument("csvs", nargs="+")
    q.add_argument("--cmd", action="append", required=True)
    q.add_argument("--kernel", default="fused_qknorm_kernel<qkn::Bf16, 4, true, 2, 512, 0, true, false>")
    q.add_argument("--title", default="fused prefill kernel (T=16384, Q and K width 5120, bf16, N=2)")
    a = ap.parse_args()
    if a.what == "sq":
        summarize_sq(a.csvs, a.out_txt, a.cmd, a.kernel, a.title)
    elif a.what == "trace":
        window = a.window or (bench_window(a.bench_json, a.leg, a.kernel) if a.bench_json else "")
        summarize_trace(a.stats_csv, a.out_txt, a.cmd, a.note, a.kernel_trace, window)
    else:
        plan = None
        if a.plans:
            import json
            plan = json.load(open(a.plans)).get(a.leg)
        summarize_traffic(a.fetch_csv, a.write_csv, a.out_txt, a.cmd_fetch, a.cmd_write,
                          a.algorithmic_bytes, a.kernel, a.title, plan)


if __name__ == "__main__":
    main()
