"""Summaries of rocprofv3 runs of bench.py, for profiles/.

For one workload, three rocprofv3 runs of bench.py (the commands are commands(); run them from /tmp on the GPU
box) leave CSV files under one output folder:
  <out>/<workload>_kt     --kernel-trace --stats: every kernel dispatch with its GPU start / end timestamps
  <out>/<workload>_fetch  --pmc FETCH_SIZE: bytes read from HBM per dispatch (KiB), and a 1 GiB device copy
  <out>/<workload>_write  --pmc WRITE_SIZE: bytes written, the same
and bench.py's JSON line of the kernel-trace run in <out>/<workload>_kt.json.  This script prints a markdown
summary (per kernel and launch shape: calls, average / median / min / max duration; per-dispatch traffic
scaled by what the same counters read for the copy, against bench.py's algorithmic bytes) and, with
--traffic-json, writes the per-launch HBM bytes that bench.py reports as roofline.traffic, tagged with a hash
of the kernels' sources so that bench.py drops them once a kernel changes.

    python3 bench_profile.py --workload prefill --out <out> [--traffic-json profiles/traffic_prefill.json]
    python3 bench_profile.py --print-commands --workload prefill --out <out>
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_MIB = 1024
SKIP = ("--no-graph --no-trace --no-cpu-baseline --no-epilogues --no-decode --no-copy-ceiling --no-workloads")


def commands(workload, out, repo="<repo>"):
    """The rocprofv3 runs a summary is made from (run from /tmp)."""
    bound = "" if workload in ("prefill", "ep8") else " --no-bound"   # the dispatch taken apart (probes)
    b = "python3 %s/bench.py --workload %s %s%s" % (repo, workload, SKIP, bound)
    cmds = [
        "rocprofv3 --kernel-trace --stats --output-format csv -d %s/%s_kt -o kt -- %s --steps 50 --warmup 10 "
        "> %s/%s_kt.json" % (out, workload, b, out, workload),
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s/%s_fetch -o fetch -- %s --steps 2 --warmup 1 "
        "--calib-copy-mib %d" % (out, workload, b, COPY_MIB),
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s/%s_write -o write -- %s --steps 2 --warmup 1 "
        "--calib-copy-mib %d" % (out, workload, b, COPY_MIB),
    ]
    if workload == "prefill":   # the step's eager launches and its graph replays (bench.py's default order)
        g = "python3 %s/bench.py --workload %s %s --no-bound" % (repo, workload, SKIP.replace("--no-graph ", ""))
        cmds.append("rocprofv3 --kernel-trace --output-format csv -d %s/%s_ktg -o ktg -- %s --steps 50 --warmup 10 "
                    "> %s/%s_ktg.json" % (out, workload, g, out, workload))
    return cmds


def _rows(folder, suffix):
    files = sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True))
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _get(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(names)


def short_name(name):
    m = re.search(r"\b(k_\w+?)(?:<([^>]*)>)?\(", name)
    if m:
        return m.group(1) + ("<%s>" % m.group(2) if m.group(2) else "")
    if "rocclr_copyBuffer" in name:          # the runtime's device-to-device copy (the calibration copy)
        return "copy:rocclr"
    return name.split("(")[0][-48:]


def _blocks(row):
    grid = int(_get(row, "Grid_Size_X", "Grid_Size", "Grid_Size_x"))
    wg = int(_get(row, "Workgroup_Size_X", "Workgroup_Size", "Workgroup_Size_x"))
    return grid // max(wg, 1), wg


def kernel_trace(folder):
    """[(kernel, blocks, threads per block, duration us, start ns)] in start order."""
    out = []
    for r in _rows(folder, "kernel_trace.csv"):
        s, e = int(_get(r, "Start_Timestamp")), int(_get(r, "End_Timestamp"))
        nb, wg = _blocks(r)
        out.append((short_name(_get(r, "Kernel_Name")), nb, wg, (e - s) / 1e3, s))
    return sorted(out, key=lambda x: x[4])


def counters(folder, counter):
    """{(kernel, blocks): [per-dispatch value]} for one counter."""
    out = {}
    for r in _rows(folder, "counter_collection.csv"):
        if _get(r, "Counter_Name") != counter:
            continue
        grid = int(_get(r, "Grid_Size"))
        wg = int(_get(r, "Workgroup_Size"))
        key = (short_name(_get(r, "Kernel_Name")), grid // max(wg, 1))
        out.setdefault(key, []).append(float(_get(r, "Counter_Value")))
    return out


def _stats(v):
    return dict(calls=len(v), avg=sum(v) / len(v), median=statistics.median(v), min=min(v), max=max(v))


def summarize(workload, out, traffic_json=None):
    import bench

    kt = kernel_trace(os.path.join(out, "%s_kt" % workload))
    try:
        with open(os.path.join(out, "%s_kt.json" % workload)) as f:
            line = json.loads(f.read().strip().splitlines()[-1])
    except (OSError, ValueError, IndexError):
        line = None
    lines = ["# Kernel trace and HBM traffic: %s" % (line["config"]["workload"] if line else workload), "",
             "Commands (one MI355X, run from /tmp; `<repo>` is the repository root, `<out>` an output folder), "
             "then `python3 <repo>/bench_profile.py --workload %s --out <out>`:" % workload, ""]
    lines += ["    " + c for c in commands(workload, "<out>")]
    lines += ["", "## rocprofv3 --kernel-trace: duration per launch shape (us)", "",
              "| kernel | blocks x threads | calls | avg | median | min | max |", "|---|---|---|---|---|---|---|"]
    groups = {}
    for name, nb, wg, d, _ in kt:
        groups.setdefault((name, nb, wg), []).append(d)
    for (name, nb, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        if name.startswith("copy:") or not name.startswith("k_"):
            continue
        s = _stats(v)
        lines.append("| %s | %d x %d | %d | %.2f | %.2f | %.2f | %.2f |" % (name, nb, wg, s["calls"], s["avg"],
                                                                       s["median"], s["min"], s["max"]))
    # the same launches split by the kernel that ran just before (a call timed back to back follows itself;
    # inside a step it follows the previous call's kernel)
    prev = {}
    for i, (name, nb, wg, d, _) in enumerate(kt):
        if not name.startswith("k_"):
            continue
        p = kt[i - 1][0] if i > 0 else "-"
        prev.setdefault((name, nb, wg, p), []).append(d)
    lines += ["", "By the kernel just before (groups of at least 10 launches):", "",
              "| kernel | blocks x threads | after | calls | avg | median |", "|---|---|---|---|---|---|"]
    for (name, nb, wg, p), v in sorted(prev.items(), key=lambda kv: -sum(kv[1])):
        if len(v) >= 10:
            lines.append("| %s | %d x %d | %s | %d | %.2f | %.2f |" % (name, nb, wg, p, len(v), sum(v) / len(v),
                                                                     statistics.median(v)))
    # eager steps against graph replays: bench.py runs W + K eager steps, then W + K replays of the step graph,
    # so the step's kernels occur in that order; the warm-ups of each are left out
    ktg = kernel_trace(os.path.join(out, "%s_ktg" % workload))
    try:
        with open(os.path.join(out, "%s_ktg.json" % workload)) as f:
            gline = json.loads(f.read().strip().splitlines()[-1])
    except (OSError, ValueError, IndexError):
        gline = None
    if ktg and gline:
        W, K = gline["warmup"], gline["steps"]
        lines += ["", "Eager steps against HIP-graph replays of the same step (4th command; %d warm-ups of each "
                  "left out): step %.1f us eager (host clock), %.1f us per graph replay." % (
                      W, gline["ms_per_step"] * 1e3, gline["step_graph_replay_us"] or 0.0), "",
                  "| kernel | blocks | eager avg | eager median | graph avg | graph median |",
                  "|---|---|---|---|---|---|"]
        seq = {}
        for name, nb, wg, d, _ in ktg:
            seq.setdefault((name, nb), []).append(d)
        for (name, nb), v in sorted(seq.items(), key=lambda kv: -sum(kv[1])):
            if not name.startswith("k_") or len(v) < 2 * (W + K):
                continue
            eager, graph = v[W:W + K], v[2 * W + K:2 * (W + K)]
            lines.append("| %s | %d | %.2f | %.2f | %.2f | %.2f |" % (name, nb, sum(eager) / K, statistics.median(eager),
                                                                    sum(graph) / K, statistics.median(graph)))
    lines += ["", "Kernel sources profiled (sha256, first 16 hex digits, as bench.py tags counter figures): " +
              ", ".join("%s %s" % (k, bench.source_hash(v)) for k, v in bench.KERNEL_SOURCES.items())]
    if line:
        calls = line["kernels"]
        lines += ["", "bench.py in the same run (HIP events around 50 back-to-back launches of each call, us): " +
                  ", ".join("%s %.2f" % (k, v["us"]) for k, v in calls.items()) +
                  "; eager step %.1f us; roofline kernel %s, avg_launch_us %.2f, frac %.4f." % (
                      line["ms_per_step"] * 1e3, line["roofline"]["kernel"], line["roofline"]["avg_launch_us"],
                      line["roofline"]["frac"])]
        b = line.get("dispatch_bound")
        if b:
            lines += ["", "The dispatch taken apart in the same run (bench.py `dispatch_bound`, events, us): its stores "
                      "alone %.2f (%.1f MB, %.0f GB/s), its source reads alone %.2f (%.1f MB, %.0f GB/s), their sum "
                      "%.2f; the dispatch %.2f." % (b["write_only_us"], b["write_bytes"] / 1e6, b["write_only_GBps"],
                                                    b["read_only_us"], b["read_bytes"] / 1e6, b["read_only_GBps"],
                                                    b["sum_us"], b["dispatch_us"])]
        c = line.get("combine_bound")
        if c:
            lines += ["", "The combine taken apart in the same run (bench.py `combine_bound`, events, us): its gathers "
                      "alone %.2f (%.1f MB, %.0f GB/s), its output writes alone %.2f (%.1f MB, %.0f GB/s), their sum "
                      "%.2f; the combine %.2f." % (c["gathers_only_us"], c["gather_bytes"] / 1e6, c["gathers_only_GBps"],
                                                   c["writes_only_us"], c["write_bytes"] / 1e6, c["writes_only_GBps"],
                                                   c["sum_us"], c["combine_us"])]

    fetch = counters(os.path.join(out, "%s_fetch" % workload), "FETCH_SIZE")
    write = counters(os.path.join(out, "%s_write" % workload), "WRITE_SIZE")
    copy_f = [v for (k, _), vs in fetch.items() if k.startswith("copy:") for v in vs]
    copy_w = [v for (k, _), vs in write.items() if k.startswith("copy:") for v in vs]
    traffic = {}
    if copy_f and copy_w:
        cb = COPY_MIB << 20
        ff = cb / (max(copy_f) * 1024.0)
        wf = cb / (max(copy_w) * 1024.0)
        lines += ["", "## HBM traffic per dispatch (rocprofv3 --pmc, one counter per run)", "",
                  "Calibration: a %d MiB device-to-device copy reads FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB, "
                  "so FETCH_SIZE is scaled by %.3f and WRITE_SIZE by %.3f to get bytes." % (
                      COPY_MIB, max(copy_f), max(copy_w), ff, wf), "",
                  "| kernel | blocks | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | written MB | total MB |",
                  "|---|---|---|---|---|---|---|"]
        for key in sorted(set(fetch) & set(write), key=lambda k: -statistics.mean(fetch[k])):
            name, nb = key
            if not name.startswith("k_"):
                continue
            fk, wk = statistics.mean(fetch[key]), statistics.mean(write[key])
            rd, wr = fk * 1024 * ff, wk * 1024 * wf
            lines.append("| %s | %d | %.1f | %.1f | %.2f | %.2f | %.2f |" % (name, nb, fk, wk, rd / 1e6, wr / 1e6,
                                                                           (rd + wr) / 1e6))
            traffic.setdefault(name.split("<")[0], []).append(dict(blocks=nb, fetch_kib=fk, write_kib=wk,
                                                                   read_bytes=int(rd), write_bytes=int(wr),
                                                                   hbm_bytes_per_launch=int(rd + wr)))
        if line:
            bm = {k: v.get("bytes") for k, v in line["kernels"].items()}
            lines += ["", "Algorithmic bytes (bench.py's byte model, this workload): " +
                      ", ".join("%s %.2f MB" % (k, b / 1e6) for k, b in bm.items() if b)]
    text = "\n".join(lines) + "\n"
    if traffic_json and traffic and line:
        kern = {}
        main = {"k_dispatch_fp8": "dispatch", "k_combine": "combine"}
        for kname, call in main.items():
            ents = traffic.get(kname)
            if not ents:
                continue
            alg = line["kernels"][call]["bytes"]
            best = min(ents, key=lambda e: abs(e["hbm_bytes_per_launch"] - alg))   # the call's own launch shape
            kern[kname] = dict(best, algorithmic_bytes=alg, ratio=round(best["hbm_bytes_per_launch"] / alg, 4),
                               source_sha256_16=bench.source_hash(bench.KERNEL_SOURCES[kname]))
        with open(traffic_json, "w") as f:
            json.dump(dict(workload=workload, calibration=dict(fetch_factor=ff, write_factor=wf,
                                                               copy_bytes=COPY_MIB << 20), kernels=kern), f,
                      indent=1)
    return text


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json")
    ap.add_argument("--print-commands", action="store_true")
    ap.add_argument("--repo", default="<repo>")
    a = ap.parse_args()
    if a.print_commands:
        print("\n".join(commands(a.workload, a.out, a.repo)))
        return
    sys.stdout.write(summarize(a.workload, a.out, a.traffic_json))


if __name__ == "__main__":
    main()
