"""Benchmark of the MoE expert-parallel layout / dispatch / combine path on one MI355X.

A step is one pass of the whole path over one batch of the prefill workload: the layout and the FP8 dispatch
with zero padding (one ep_layout_dispatch call: the layout kernels, then the dispatch), then the weighted BF16
combine (4096 tokens, hidden 7168, 256 experts in 8 groups with group-limited top-4-group / top-8 routing,
alignment 128).  Inputs and expert outputs are resident in HBM before timing
starts.  W untimed warm-up steps, then exactly K timed steps bracketed by device syncs; the host enqueues the
calls of a step far faster than the GPU runs them, so no step waits on the host.  The same step captured in a
HIP graph and replayed K times is reported too (`step_graph_replay_us`).

Per call, two timings:
  * back to back: HIP events on the launch stream around K back-to-back launches of the call;
  * flushed (the pages' method: a cache flush -- a 2 GiB read sweep -- before every sample, 10 warm-up + 50
    samples): each sample's kernels timed by their GPU start/end timestamps from a kernel trace (torch's
    profiler), so nothing is inserted between a flush and the call after it.  Median and min.

Prints one JSON line.  `value` is the step's effective HBM throughput: the algorithmic bytes of layout +
dispatch + combine per step divided by the measured step time.  Algorithmic bytes are what the method must
move: every token row read once, every routed row written once, padding rows when zero padding is requested,
the expert rows gathered once by combine and the output written once (bytes_model()).  `roofline` is for the
dominant kernel, `cpu_baseline` the oracle timed on the host (one pinned core, and all cores over token
ranges).  `workloads` has every workload (tiny, decode, prefill, ep8, skewed) measured the same way;
`dispatch_bound` times the prefill dispatch's write stream and read stream on their own, `combine_bound` the
prefill combine's gathers and output writes on their own (bench_probe.hip).
`step_kernels_us` gives each kernel's GPU time inside the step (a kernel trace of K more eager steps), and
`roofline.frac_in_step` the dominant kernel's rate there.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X published HBM3E peak
WORKLOAD = "prefill"
ALL_WORKLOADS = ("tiny", "decode", "prefill", "ep8", "skewed")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill.json")
PROBE_LIB = os.path.join(ROOT, "libbench_probe.so")
FLUSH_BYTES = 2 << 30         # the flush reads 2 GiB: more than the memory-side cache and every L2
# the source files each kernel is compiled from (their hash marks counter figures taken from an older kernel)
KERNEL_SOURCES = {
    "k_dispatch_fp8": ("ep_dispatch.hip", "ep_dispatch_core.hpp", "ep_device.hpp"),
    "k_combine": ("ep_combine.hip", "ep_device.hpp"),
    "layout": ("ep_layout.hip", "ep_layout_core.hpp", "ep_device.hpp"),
    "k_layout_dispatch_small": ("ep_fused.hip", "ep_layout_core.hpp", "ep_dispatch_core.hpp", "ep_device.hpp"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the steps (counter calibration)")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-epilogues", dest="epilogues", action="store_false",
                    help="skip the receiver-placement / source-reduce measurement at the EP8 shapes")
    ap.add_argument("--no-workloads", dest="workloads", action="store_false",
                    help="skip the per-call table of the other workloads (tiny, decode, ep8, skewed)")
    ap.add_argument("--no-copy-ceiling", dest="copy_ceiling", action="store_false",
                    help="skip the timed plain device copy reported as context")
    ap.add_argument("--no-decode", dest="decode", action="store_false",
                    help="skip the decode-shape comparison of the one-launch layout + dispatch")
    ap.add_argument("--no-flushed", dest="flushed", action="store_false",
                    help="skip the flushed (pages' method) timings")
    ap.add_argument("--no-bound", dest="bound", action="store_false",
                    help="skip the dispatch write-stream / read-stream probes")
    ap.add_argument("--no-trace", dest="trace", action="store_false",
                    help="no in-process kernel trace (no flushed timings, no step_kernels_us): for runs under rocprofv3")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the HIP-graph replay of the step (a kernel trace then holds eager launches only)")
    a = ap.parse_args()
    if not a.trace:
        a.flushed = False
    return a


def bytes_model(cfg, counts):
    """Algorithmic bytes of each operation for one step.  counts: V (valid local rows), P (padding rows),
    N_send (send-window rows)."""
    T, H, K, E, R = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks
    El = E // R
    V, P, S = counts["V"], counts["P"], counts["N_send"]
    row_b = (H + 4 * (H // 128)) if cfg.fp8 else 2 * H
    layout = T * K * 8 + T * K * 4 + T * R + 4 * (E + R + El + 2) + (T * R * 4 if R > 1 else 0)
    dispatch = (T * 2 * H                      # x, read once
                + T * K * 4 + T * K * 4        # slot map + routing weights
                + (T * R * 4 if R > 1 else 0)  # send slots
                + V * (row_b + 8)              # routed rows + row metadata (src idx, weight)
                + P * 8 + (P * row_b if cfg.zero_padding else 0)
                + S * (row_b + 4 + K * 12))    # send rows + src idx + topk idx (int64) / weight
    combine = V * 2 * H + T * K * 8 + T * 2 * H + (T * 2 * H if cfg.bias else 0)
    return dict(layout=layout, dispatch=dispatch, combine=combine, row_bytes=row_b)


def source_hash(fnames):
    h = hashlib.sha256()
    for fname in fnames:
        with open(os.path.join(ROOT, "combine_get_dispatch_03_amd", "csrc", fname), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return k.get("hbm_bytes_per_launch")


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---- the oracle on the host (cpu_baseline) -----------------------------------------------------------------

def cpu_baseline(inp, y_bits, cfg):
    """The oracle as it stands on the full workload.  (i) One thread pinned to one host core: layout, dispatch
    and combine, repeated until about 10 s of CPU time (at least 3 runs), the median run.  (ii) All the host
    cores this process may use: the layout once (serial), then the same C dispatch and combine functions over
    contiguous token ranges, one thread per core (the calls release the GIL); zero padding is written by the
    first range only, so every row is written once; the median of 3 runs."""
    import numpy as np

    import oracle as O
    import workloads as W

    idx = np.ascontiguousarray(inp["topk_idx"].numpy())
    w = np.ascontiguousarray(inp["topk_weights"].numpy())
    x = np.ascontiguousarray(W.bf16_bits(inp["x"]))
    bias = W.bf16_bits(inp["bias"]) if inp["bias"] is not None else None
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    El = cfg.num_experts // cfg.num_ranks

    def one_pass():
        lay = O.layout(idx, cfg.num_experts, cfg.num_ranks, cfg.rank, cfg.expert_alignment)
        O.dispatch(x, idx, w, lay, cfg.num_experts, cfg.num_ranks, cfg.rank, cfg.expert_alignment, fp8=cfg.fp8,
                   zero_pad=cfg.zero_padding, recv_fill=None)
        O.combine(y_bits, lay["slot"], w, bias)
        return lay

    os.sched_setaffinity(0, {core})
    times = []
    try:
        while len(times) < 3 or sum(times) < 10.0:
            t0 = time.perf_counter()
            lay = one_pass()
            times.append(time.perf_counter() - t0)
    finally:
        os.sched_setaffinity(0, set(allowed))
    cnt = lay["cnt"][cfg.rank * El:(cfg.rank + 1) * El]
    V = int(cnt.sum())
    counts = dict(V=V, P=int(lay["psum"][-1]) - V, N_send=int(sum(lay["ntok_rank"][r] for r in range(cfg.num_ranks)
                                                                    if r != cfg.rank)))
    bm = bytes_model(cfg, counts)
    total = bm["layout"] + bm["dispatch"] + bm["combine"]
    med = float(np.median(times))

    # (ii) all cores: token ranges
    ncores = len(allowed)
    if cfg.num_ranks == 1:
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            _, t_lay = oracle_token_ranges(x, idx, w, y_bits, bias, cfg, ncores)
            runs.append((t_lay, time.perf_counter() - t0))
        med_all = sorted(b for _, b in runs)[1]
        all_cores = dict(value=round(total / med_all / 1e9, 3), unit="GB/s", cores=ncores, kind="oracle",
                         sample="full %s workload, layout serial (%.2f ms) then dispatch + combine over %d token "
                                "ranges on %d threads; median of 3 runs, %.3f s each"
                                % (cfg.name, 1e3 * float(np.median([a for a, _ in runs])), ncores, ncores, med_all))
    else:
        all_cores = None
    return dict(value=round(total / med / 1e9, 3), unit="GB/s", cores=1, kind="oracle",
                sample="full %s workload (layout + FP8 dispatch + combine), one thread pinned to one core, median "
                       "of %d runs, %.2f s each" % (cfg.name, len(times), med),
                pinned_core=core, host_cores_available=len(allowed), host_cpu=host_cpu_model(),
                all_cores=all_cores)


def oracle_token_ranges(x, idx, w, y_bits, bias, cfg, ncores):
    """The oracle's layout (serial), then its C dispatch and combine functions over `ncores` contiguous token
    ranges, one thread each (ctypes releases the GIL inside the calls).  One rank only (the send windows' rows
    depend on the whole batch).  Zero padding is written by the first range only, so every row is written
    once.  Returns (dict of outputs, layout seconds)."""
    import concurrent.futures

    import numpy as np

    import oracle as O

    assert cfg.num_ranks == 1
    lib, P = O._load(), O._ptr
    T, H, K = cfg.num_tokens, cfg.hidden, cfg.num_topk
    G = H // 128 if cfg.fp8 else 0
    rowb = H if cfg.fp8 else 2 * H
    t0 = time.perf_counter()
    lay = O.layout(idx, cfg.num_experts, 1, 0, cfg.expert_alignment)
    t_lay = time.perf_counter() - t0
    cap = lay["cap"]
    o = dict(recv_x=np.zeros((cap, rowb), np.uint8), recv_scales=np.zeros((cap, max(G, 1)), np.float32),
             recv_src=np.full(cap, -7, np.int32), recv_w=np.full(cap, -7.0, np.float32),
             out=np.empty((T, H), np.float64), lay=lay)
    slot = lay["slot"]
    bounds = [(T * i // ncores, T * (i + 1) // ncores) for i in range(ncores)]

    def part(i):
        a, b = bounds[i]
        if b <= a and not (i == 0 and cfg.zero_padding):
            return
        rc = lib.oracle_dispatch(P(x[a:b]), b - a, H, K, P(w[a:b]), P(idx[a:b]), cfg.num_experts, 1, 0,
                                 cfg.expert_alignment, int(cfg.fp8), int(cfg.zero_padding and i == 0), 1,
                                 P(lay["cnt"]), P(lay["psum"]), P(slot[a:b]), P(lay["send_slot"][a:b]),
                                 P(o["recv_x"]), P(o["recv_scales"]) if G else None, P(o["recv_src"]),
                                 P(o["recv_w"]), None, None, None, None, None, None)
        if rc != 0:
            raise ValueError("oracle_dispatch rejected a token range")
        if a > 0:   # the call numbers its tokens from the start of its range
            rows = slot[a:b].ravel()
            o["recv_src"][rows[rows >= 0]] += a
        lib.oracle_combine(P(y_bits), H, P(slot[a:b]), P(w[a:b]), b - a, K,
                           P(bias[a:b]) if bias is not None else None, P(o["out"][a:b]))

    with concurrent.futures.ThreadPoolExecutor(ncores) as ex:
        list(ex.map(part, range(ncores)))
    return o, t_lay


# ---- GPU timing helpers -------------------------------------------------------------------------------------

class Probe:
    """bench_probe.hip: the flush used between flushed samples and the dispatch's write-stream / read-stream
    probes.  Launches go to torch's current stream."""

    def __init__(self, dev):
        import torch
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError("libbench_probe.so is not built: run __graft_entry__.build()")
        self.lib = ctypes.CDLL(PROBE_LIB)
        Pt, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        self.lib.probe_flush.restype = I
        self.lib.probe_flush.argtypes = [Pt, I64, Pt, Pt]
        self.lib.probe_dispatch_writes.restype = I
        self.lib.probe_dispatch_writes.argtypes = [Pt, I, I, Pt, I, Pt, Pt, Pt, Pt, I, Pt]
        self.lib.probe_dispatch_reads.restype = I
        self.lib.probe_dispatch_reads.argtypes = [Pt, Pt, I, I, I, Pt, Pt]
        self.lib.probe_copy.restype = I
        self.lib.probe_copy.argtypes = [Pt, Pt, I64, Pt]
        self.lib.probe_send_writes.restype = I
        self.lib.probe_send_writes.argtypes = [Pt, Pt, I, I, I, Pt, Pt, Pt, Pt, Pt, Pt, Pt, I, Pt]
        self.lib.probe_combine_gathers.restype = I
        self.lib.probe_combine_gathers.argtypes = [Pt, Pt, I, I, I, Pt, Pt]
        self.lib.probe_row_writes.restype = I
        self.lib.probe_row_writes.argtypes = [Pt, I, I, Pt]
        self.junk = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev).fill_(3)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)

    @staticmethod
    def _stream():
        import torch
        return torch.cuda.current_stream().cuda_stream

    def flush(self):
        rc = self.lib.probe_flush(self.junk.data_ptr(), self.junk.numel(), self.sink.data_ptr(), self._stream())
        if rc != 0:
            raise RuntimeError("probe_flush failed (%d)" % rc)

    def copy(self, src, dst):
        rc = self.lib.probe_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), self._stream())
        if rc != 0:
            raise RuntimeError("probe_copy failed (%d)" % rc)


def events_us(fn, n):
    """Average µs of fn over n back-to-back calls, HIP events on the launch stream around them (the GPU first spins
    ~20 ms so that the host enqueues every call before the first runs)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * 0.02))
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def flushed_us(fn, probe, warmup=10, samples=50):
    """The pages' method: a cache flush before every sample, 10 warm-up samples, then 50 timed ones, each timed
    by the GPU's own start and end timestamps of its kernels from a kernel trace (torch's profiler, which
    records every kernel dispatched in the process), so nothing is inserted between a flush and the call after
    it.  A sample's time is the sum of its kernels' durations (the gaps between a call's own kernels, a launch
    gap each, are not in it).  Returns (median, min) in µs."""
    import numpy as np
    import torch
    from torch.profiler import ProfilerActivity, profile

    for _ in range(warmup):
        probe.flush()
        fn()
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(samples):
            probe.flush()
            fn()
        torch.cuda.synchronize()
    evs = sorted((e for e in prof.events() if e.device_type == torch.autograd.DeviceType.CUDA),
                 key=lambda e: e.time_range.start)
    per = []
    for e in evs:
        if "k_probe_flush" in e.name:
            per.append(0.0)
        elif per:
            per[-1] += e.time_range.end - e.time_range.start
    if len(per) != samples or min(per) <= 0.0:
        raise RuntimeError("flushed timing: %d samples traced, expected %d" % (len(per), samples))
    return float(np.median(per)), float(np.min(per))


def traced_kernels_us(fn, n):
    """GPU duration of every kernel fn launches, from a kernel trace (torch's profiler) of n calls: {kernel name:
    average µs}, names shortened to the kernel's own identifier."""
    import re

    import torch
    from torch.profiler import ProfilerActivity, profile

    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
    out = {}
    for e in prof.events():
        if e.device_type != torch.autograd.DeviceType.CUDA:
            continue
        m = re.search(r"\b(k_\w+?)(?:<[^>]*>)?\(", e.name)
        out.setdefault(m.group(1) if m else e.name[:40], []).append(e.time_range.end - e.time_range.start)
    return {k: round(sum(v) / len(v), 2) for k, v in out.items()}


def rate(b, us):
    return b / (us * 1e-6) / 1e9


def progress(msg):
    print("[bench] %s" % msg, file=sys.stderr, flush=True)


# ---- per-workload table -------------------------------------------------------------------------------------

def measure_workload(ep, W, dev, name, n, probe, flushed=True):
    """One workload measured per call (layout, dispatch, combine, layout + dispatch as two calls and as one call):
    back to back and flushed; algorithmic bytes and GB/s against the median; tokens/s = T / median; padding
    amplification A_pad (rows used / valid rows) and max / mean rows per local expert; and the eager step
    (one-call layout + dispatch, then combine), the median of five blocks of n steps between device syncs."""
    import numpy as np
    import torch

    inp = W.make_inputs(name)
    cfg = inp["cfg"]
    T, K, E, R, A = cfg.num_tokens, cfg.num_topk, cfg.num_experts, cfg.num_ranks, cfg.expert_alignment
    idx = inp["topk_idx"].to(dev)
    w = inp["topk_weights"].to(dev)
    x = inp["x"].to(dev)
    bias = inp["bias"].to(dev) if inp["bias"] is not None else None
    ws = torch.empty(ep.ep_layout_workspace_bytes(T, K, E, R, A), dtype=torch.uint8, device=dev)
    lay = dict(num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=dev),
               num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=dev),
               is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=dev),
               psum_num_recv_tokens_per_expert=torch.empty(E // R + 1, dtype=torch.int32, device=dev),
               num_invalid_topk=torch.empty(1, dtype=torch.int32, device=dev))
    h, _ = ep.ep_get_layout(idx, E, R, cfg.rank, A, workspace=ws, outputs=lay)
    dout = ep.alloc_dispatch_outputs(h, cfg.hidden, cfg.fp8, device=dev)
    y = W.random_expert_outputs(h.recv_capacity, cfg.hidden, seed=1234, device=dev)
    res = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device=dev)

    calls = {
        "layout": lambda: ep.ep_get_layout(idx, E, R, cfg.rank, A, workspace=ws, outputs=lay),
        "dispatch": lambda: ep.ep_dispatch(h, x, w, fp8=cfg.fp8, do_zero_padding=cfg.zero_padding, out=dout),
        "combine": lambda: ep.ep_combine(h, y, w, bias, out=res),
    }

    def two_calls():
        hh, _ = ep.ep_get_layout(idx, E, R, cfg.rank, A, workspace=ws, outputs=lay)
        ep.ep_dispatch(hh, x, w, fp8=cfg.fp8, do_zero_padding=cfg.zero_padding, out=dout)

    def one_call():
        ep.ep_layout_dispatch(idx, x, E, R, cfg.rank, A, w, fp8=cfg.fp8, do_zero_padding=cfg.zero_padding,
                              out=dout, workspace=ws, outputs=lay)

    calls["layout_then_dispatch"] = two_calls
    calls["layout_dispatch_one_call"] = one_call

    def step():
        hs, _, _ = ep.ep_layout_dispatch(idx, x, E, R, cfg.rank, A, w, fp8=cfg.fp8,
                                         do_zero_padding=cfg.zero_padding, out=dout, workspace=ws, outputs=lay)
        ep.ep_combine(hs, y, w, bias, out=res)

    for fn in calls.values():
        fn()
    torch.cuda.synchronize()
    cnt = lay["num_tokens_per_expert"].cpu().numpy()
    psum = lay["psum_num_recv_tokens_per_expert"].cpu().numpy()
    ntr = lay["num_tokens_per_rank"].cpu().numpy()
    El = E // R
    cl = cnt[cfg.rank * El:(cfg.rank + 1) * El]
    V = int(cl.sum())
    counts = dict(V=V, P=int(psum[-1]) - V, N_send=int(sum(ntr[r] for r in range(R) if r != cfg.rank)))
    bm = bytes_model(cfg, counts)
    bm["layout_then_dispatch"] = bm["layout"] + bm["dispatch"]
    bm["layout_dispatch_one_call"] = bm["layout_then_dispatch"]

    out = dict(workload=describe(cfg), tokens=T, valid_rows=V, pad_rows=counts["P"], send_rows=counts["N_send"],
               A_pad=round(int(psum[-1]) / max(V, 1), 4),
               max_mean_rows_per_expert=[int(cl.max()), round(float(cl.mean()), 2)], calls={})
    for k, fn in calls.items():
        us = events_us(fn, n)
        c = dict(us=round(us, 2), bytes=bm[k])
        if flushed:
            fmed, fmin = flushed_us(fn, probe)
            c.update(us_flushed_median=round(fmed, 2), us_flushed_min=round(fmin, 2))
        ref = c.get("us_flushed_median", us)
        c["tokens_per_s"] = round(T / (ref * 1e-6), 1)
        if k != "layout":
            c["GBps"] = round(rate(bm[k], us), 1)
            c["pct_peak"] = round(100 * rate(bm[k], us) / HBM_PEAK_GBPS, 1)
            if flushed:
                c["GBps_flushed"] = round(rate(bm[k], c["us_flushed_median"]), 1)
                c["pct_peak_flushed"] = round(100 * rate(bm[k], c["us_flushed_median"]) / HBM_PEAK_GBPS, 1)
        out["calls"][k] = c
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    blocks = []
    for _ in range(5):
        t0 = time.perf_counter()
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        blocks.append((time.perf_counter() - t0) * 1e6 / n)
    step_us = float(np.median(blocks))
    out["step_us"] = round(step_us, 2)
    out["step_GBps"] = round(rate(bm["layout"] + bm["dispatch"] + bm["combine"], step_us), 1)
    h.free()
    del ws, lay, dout, y, res, idx, w, x, bias
    torch.cuda.empty_cache()
    return out


def describe(cfg):
    return ("%s: %d tok x hidden %d, %d experts%s, top-%d, %s dispatch%s, BF16 combine%s, alignment %d%s" % (
        cfg.name, cfg.num_tokens, cfg.hidden, cfg.num_experts,
        " (8 groups, top-4 groups)" if cfg.routing == "grouped" else
        (" (Zipf %.1f)" % cfg.zipf_s if cfg.routing == "zipf" else ""), cfg.num_topk,
        "FP8 e4m3 per-128" if cfg.fp8 else "BF16", " + zero padding" if cfg.zero_padding else "",
        " + bias" if cfg.bias else "", cfg.expert_alignment,
        ", %d ranks (rank %d), %d send windows" % (cfg.num_ranks, cfg.rank, cfg.num_ranks - 1)
        if cfg.num_ranks > 1 else ""))


# ---- the prefill dispatch's write stream and read stream on their own ---------------------------------------

def measure_dispatch_bound(ep, W, dev, n, probe):
    """The FP8 dispatch with zero padding on the prefill workload, taken apart:
    * the dispatch's stores alone (probe_dispatch_writes: the same destination rows, scales, row metadata and
      padding rows, in the same work split, no reads) and its source reads alone (probe_dispatch_reads: the
      token rows and the slot map, no stores).  Both use the dispatch's own load and store kinds.  When both
      streams come from HBM their sum bounds the dispatch from below (reads and writes share each channel's
      data bus); back to back, the source rows come from the memory-side cache instead;
    * the product dispatch without zero padding (routed rows only) and with alignment 1 (no padding rows at
      all), and the increment that zero padding adds."""
    import torch

    inp = W.make_inputs("prefill")
    cfg = inp["cfg"]
    T, K, E, A, H = cfg.num_tokens, cfg.num_topk, cfg.num_experts, cfg.expert_alignment, cfg.hidden
    G = H // 128
    idx, w, x = inp["topk_idx"].to(dev), inp["topk_weights"].to(dev), inp["x"].to(dev)
    h, lay = ep.ep_get_layout(idx, E, 1, 0, A)
    d = ep.ep_dispatch(h, x, w, fp8=True, do_zero_padding=True)
    torch.cuda.synchronize()
    used = int(lay["psum_num_recv_tokens_per_expert"][-1].item())
    token_rows, V, pads = local_rows_by_token(d["recv_src_idx"].cpu().numpy(), used, T, K)
    tr = torch.from_numpy(token_rows).to(dev)
    pr = torch.from_numpy(pads).to(dev) if pads.size else torch.zeros(1, dtype=torch.int32, device=dev)
    lib, stream = probe.lib, probe._stream

    def writes():
        rc = lib.probe_dispatch_writes(tr.data_ptr(), T, K, pr.data_ptr(), int(pads.size), d["recv_x"].data_ptr(),
                                       d["recv_x_scales"].data_ptr(), d["recv_src_idx"].data_ptr(),
                                       d["recv_topk_weights"].data_ptr(), H, stream())
        assert rc == 0, rc

    def reads():
        rc = lib.probe_dispatch_reads(x.data_ptr(), tr.data_ptr(), T, K, H, probe.sink.data_ptr(), stream())
        assert rc == 0, rc

    P = pads.size
    wbytes = (V + P) * (H + 4 * G + 8)
    rbytes = T * 2 * H + T * K * 4
    full = lambda: ep.ep_dispatch(h, x, w, fp8=True, do_zero_padding=True, out=d)
    routed = lambda: ep.ep_dispatch(h, x, w, fp8=True, do_zero_padding=False, out=d)
    h1, _ = ep.ep_get_layout(idx, E, 1, 0, 1)
    d1 = ep.ep_dispatch(h1, x, w, fp8=True)
    no_pad = lambda: ep.ep_dispatch(h1, x, w, fp8=True, out=d1)
    us = {k: events_us(f, n) for k, f in (("writes", writes), ("reads", reads), ("dispatch", full),
                                          ("routed_only", routed), ("alignment_1", no_pad))}
    bm = bytes_model(cfg, dict(V=V, P=P, N_send=0))
    s = us["writes"] + us["reads"]
    pad_bytes = P * (H + 4 * G)
    h.free()
    h1.free()
    return dict(
        note="prefill FP8 dispatch with zero padding: its stores alone and its source reads alone "
             "(bench_probe.hip, same destination rows and work split), back to back, events; bound_* price "
             "the dispatch's bytes on the sum of the two",
        write_only_us=round(us["writes"], 2), write_bytes=wbytes, write_only_GBps=round(rate(wbytes, us["writes"]), 1),
        read_only_us=round(us["reads"], 2), read_bytes=rbytes, read_only_GBps=round(rate(rbytes, us["reads"]), 1),
        sum_us=round(s, 2), dispatch_us=round(us["dispatch"], 2), dispatch_bytes=bm["dispatch"],
        bound_GBps=round(rate(bm["dispatch"], s), 1),
        bound_pct_peak=round(100 * rate(bm["dispatch"], s) / HBM_PEAK_GBPS, 1),
        routed_only_us=round(us["routed_only"], 2), alignment_1_us=round(us["alignment_1"], 2),
        zero_padding_increment_us=round(us["dispatch"] - us["routed_only"], 2),
        zero_padding_increment_GBps=round(rate(pad_bytes, max(us["dispatch"] - us["routed_only"], 1e-3)), 1))


# ---- context measurements -----------------------------------------------------------------------------------

def measure_epilogues(ep, W, dev, n, probe=None):
    """Receiver-side placement and source-side reduce at the EP8 shapes: rank 0 (experts 0..31 of 256) receiving
    the rows of 7 other ranks of 4096 tokens each (top-8 uniform routing, FP8 rows + 56 scales, alignment 128),
    and the reduce of 8 returned windows of 4096 x 7168 BF16 rows with the local part and a bias.  Back to back
    (events), and with a probe also flushed (the placement's 140 MB of received rows stay in the memory-side
    cache between back-to-back calls, so the flushed figure is the one with them coming from HBM)."""
    import torch

    cfg = W.CONFIGS["ep8"]
    T, H, K, E, R, A = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks, cfg.expert_alignment
    El, G = E // R, H // 128
    gen = torch.Generator().manual_seed(77)
    tk = torch.full((R * T, K), -1, dtype=torch.int64)
    tw = torch.zeros((R * T, K), dtype=torch.float32)
    n_valid = 0
    for s in range(1, R):
        idx = W.route_uniform_distinct(T, E, K, gen)
        w = W.softmax_weights(torch.randn(T, K, generator=gen))
        mine = (idx < El).any(dim=1)
        sel = torch.nonzero(mine).flatten()
        ns = sel.numel()
        loc = torch.where(idx[sel] < El, idx[sel], torch.full_like(idx[sel], -1))
        tk[s * T:s * T + ns] = loc
        tw[s * T:s * T + ns] = w[sel]
        n_valid += ns
    rows = torch.randint(0, 0x7E, (R * T, H), generator=gen, dtype=torch.uint8).to(dev)
    sc = torch.rand(R * T, G, generator=gen).to(dev)
    tk, tw = tk.to(dev), tw.to(dev)
    hr, lr = ep.ep_get_layout(tk, El, 1, 0, A)
    out = ep.ep_dispatch_rows(hr, rows, sc, tw, do_zero_padding=False)
    torch.cuda.synchronize()
    cnt = lr["num_tokens_per_expert"].cpu().numpy()
    V = int(cnt.sum())
    P = int(lr["psum_num_recv_tokens_per_expert"][-1].item()) - V
    row_b = H + 4 * G
    place = lambda: ep.ep_dispatch_rows(hr, rows, sc, tw, do_zero_padding=False, out=out)
    t_rows = events_us(place, n)
    b_rows = n_valid * row_b + R * T * K * 12 + V * (row_b + 8) + P * 8
    f_rows = flushed_us(place, probe)[0] if probe is not None else None

    inp = W.make_inputs("ep8")
    h0, l0 = ep.ep_get_layout(inp["topk_idx"].to(dev), E, R, 0, A)
    parts = W.random_expert_outputs(R * T, H, seed=3, device=dev).view(R, T, H)
    local = W.random_expert_outputs(T, H, seed=4, device=dev)
    bias = W.random_expert_outputs(T, H, seed=5, device=dev)
    red = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    reduce = lambda: ep.ep_combine_reduce(h0, parts, local, bias, out=red)
    t_red = events_us(reduce, n)
    f_red = flushed_us(reduce, probe)[0] if probe is not None else None
    ntr = l0["num_tokens_per_rank"].cpu().numpy()
    n_part = int(sum(ntr[r] for r in range(1, R)))
    b_red = n_part * 2 * H + 3 * T * 2 * H + T * R * 4
    hr.free()
    h0.free()
    res = dict(
        dispatch_rows=dict(us=round(t_rows, 2), bytes=b_rows, GBps=round(rate(b_rows, t_rows), 1),
                           received_rows=n_valid, placed_rows=V),
        combine_reduce=dict(us=round(t_red, 2), bytes=b_red, GBps=round(rate(b_red, t_red), 1),
                            partial_rows=n_part))
    for k, f, b in (("dispatch_rows", f_rows, b_rows), ("combine_reduce", f_red, b_red)):
        if f is not None:
            res[k].update(us_flushed_median=round(f, 2), GBps_flushed=round(rate(b, f), 1))
    return res


def local_rows_by_token(recv_src, used, T, K):
    """[T, K] expert-major rows of each token's local entries (in row order, -1 past them) and the padding rows,
    from the dispatch's recv_src_idx over the rows in use."""
    import numpy as np

    src = recv_src[:used]
    rows = np.nonzero(src >= 0)[0]
    pads = np.nonzero(src < 0)[0].astype(np.int32)
    toks = src[rows]
    order = np.lexsort((rows, toks))
    token_rows = np.full((T, K), -1, np.int32)
    kpos = np.zeros(T, np.int64)
    for r, t in zip(rows[order], toks[order]):
        token_rows[t, kpos[t]] = r
        kpos[t] += 1
    return token_rows, rows.size, pads


def measure_combine_bound(ep, W, dev, n, probe):
    """The weighted combine on the prefill workload, taken apart like the dispatch: its gathers alone
    (probe_combine_gathers: the same rows of y for every token, one wave per (token, 1 KiB segment), issued as the
    combine issues them, no stores) and its output stream alone (probe_row_writes: the [T, H] bf16 rows, one wave
    per (token, 1 KiB segment), nothing read), against the combine itself.  Back to back, events."""
    import torch

    inp = W.make_inputs("prefill")
    cfg = inp["cfg"]
    T, K, E, A, H = cfg.num_tokens, cfg.num_topk, cfg.num_experts, cfg.expert_alignment, cfg.hidden
    idx, w, x = inp["topk_idx"].to(dev), inp["topk_weights"].to(dev), inp["x"].to(dev)
    h, lay = ep.ep_get_layout(idx, E, 1, 0, A)
    d = ep.ep_dispatch(h, x, w, fp8=True, do_zero_padding=True)
    torch.cuda.synchronize()
    used = int(lay["psum_num_recv_tokens_per_expert"][-1].item())
    token_rows, V, _ = local_rows_by_token(d["recv_src_idx"].cpu().numpy(), used, T, K)
    tr = torch.from_numpy(token_rows).to(dev)
    y = W.random_expert_outputs(h.recv_capacity, H, seed=99, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    lib, stream = probe.lib, probe._stream

    def gathers():
        rc = lib.probe_combine_gathers(y.data_ptr(), tr.data_ptr(), T, K, H, probe.sink.data_ptr(), stream())
        assert rc == 0, rc

    def writes():
        rc = lib.probe_row_writes(out.data_ptr(), T, H, stream())
        assert rc == 0, rc

    us = {k: events_us(f, n) for k, f in (("gathers", gathers), ("writes", writes),
                                          ("combine", lambda: ep.ep_combine(h, y, w, out=out)))}
    gbytes, wbytes = V * 2 * H + T * K * 4, T * 2 * H
    h.free()
    return dict(
        note="prefill weighted combine: its gathers alone and its output writes alone (bench_probe.hip, same rows "
             "and work split), back to back, events",
        gathers_only_us=round(us["gathers"], 2), gather_bytes=gbytes,
        gathers_only_GBps=round(rate(gbytes, us["gathers"]), 1),
        writes_only_us=round(us["writes"], 2), write_bytes=wbytes, writes_only_GBps=round(rate(wbytes, us["writes"]), 1),
        sum_us=round(us["gathers"] + us["writes"], 2), combine_us=round(us["combine"], 2))


def measure_send_bound(ep, W, dev, n, probe):
    """The FP8 dispatch with send windows on the ep8 workload (rank 0 of 8, no zero padding), taken apart like the
    prefill dispatch: its stores alone (probe_send_writes: the same local expert-major rows and window rows with
    their scales, the local rows' metadata and the window rows' source index, in the same work split, no reads)
    and its source reads alone (probe_dispatch_reads: the token rows and the slot map)."""
    import numpy as np
    import torch

    inp = W.make_inputs("ep8")
    cfg = inp["cfg"]
    T, K, E, R, A, H = (cfg.num_tokens, cfg.num_topk, cfg.num_experts, cfg.num_ranks, cfg.expert_alignment,
                        cfg.hidden)
    G = H // 128
    idx, w, x = inp["topk_idx"].to(dev), inp["topk_weights"].to(dev), inp["x"].to(dev)
    h, lay = ep.ep_get_layout(idx, E, R, cfg.rank, A)
    d = ep.ep_dispatch(h, x, w, fp8=True)
    torch.cuda.synchronize()
    used = int(lay["psum_num_recv_tokens_per_expert"][-1].item())
    token_rows, V, _ = local_rows_by_token(d["recv_src_idx"].cpu().numpy(), used, T, K)
    in_rank = lay["is_token_in_rank"].cpu().numpy().astype(bool)
    send_rows = np.where(in_rank, np.cumsum(in_rank, axis=0) - 1, -1).astype(np.int32)   # row in rank r's window
    send_rows[:, cfg.rank] = -1
    S = int((send_rows >= 0).sum())
    tr = torch.from_numpy(token_rows).to(dev)
    sr = torch.from_numpy(send_rows).to(dev)
    lib, stream = probe.lib, probe._stream

    def writes():
        rc = lib.probe_send_writes(tr.data_ptr(), sr.data_ptr(), T, K, R, d["recv_x"].data_ptr(),
                                   d["recv_x_scales"].data_ptr(), d["recv_src_idx"].data_ptr(),
                                   d["recv_topk_weights"].data_ptr(), d["send_x"].data_ptr(),
                                   d["send_x_scales"].data_ptr(), d["send_src_idx"].data_ptr(), H, stream())
        assert rc == 0, rc

    def reads():
        rc = lib.probe_dispatch_reads(x.data_ptr(), tr.data_ptr(), T, K, H, probe.sink.data_ptr(), stream())
        assert rc == 0, rc

    full = lambda: ep.ep_dispatch(h, x, w, fp8=True, out=d)
    us = {k: events_us(f, n) for k, f in (("writes", writes), ("reads", reads), ("dispatch", full))}
    wbytes = V * (H + 4 * G + 8) + S * (H + 4 * G + 4)
    rbytes = T * 2 * H + T * K * 4
    bm = bytes_model(cfg, dict(V=V, P=used - V, N_send=S))
    s_us = us["writes"] + us["reads"]
    h.free()
    return dict(
        note="ep8 FP8 dispatch with 7 send windows: its stores alone and its source reads alone (bench_probe.hip, "
             "same destination rows and work split), back to back, events",
        local_rows=V, window_rows=S,
        write_only_us=round(us["writes"], 2), write_bytes=wbytes, write_only_GBps=round(rate(wbytes, us["writes"]), 1),
        read_only_us=round(us["reads"], 2), read_bytes=rbytes, read_only_GBps=round(rate(rbytes, us["reads"]), 1),
        sum_us=round(s_us, 2), dispatch_us=round(us["dispatch"], 2), dispatch_bytes=bm["dispatch"],
        bound_GBps=round(rate(bm["dispatch"], s_us), 1),
        bound_pct_peak=round(100 * rate(bm["dispatch"], s_us) / HBM_PEAK_GBPS, 1))


def measure_copy_ceiling(dev, n, probe, mib=1024):
    """A plain device-to-device copy of `mib` MiB, timed with events over n back-to-back copies: the streaming rate
    this GPU reaches on a flat read + flat write, as context for the kernels' rates (not the roofline's
    denominator, which is the published 8 TB/s).  `us` / `GBps` time a flat copy kernel (bench_probe.hip: one wave
    per 1 KiB, non-temporal 16-byte loads and stores); torch's copy_ (the runtime's copy kernel) is reported beside
    it and is slower on this chip."""
    import torch

    a = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        probe.copy(a, b)
        b.copy_(a)
    us = events_us(lambda: probe.copy(a, b), n)
    us_torch = events_us(lambda: b.copy_(a), n)
    ok = bool(torch.equal(a[:1 << 20], b[:1 << 20]))
    del a, b
    nb = 2 * (mib << 20)
    return dict(bytes_per_copy=nb, us=round(us, 2), GBps=round(rate(nb, us), 1), torch_copy_us=round(us_torch, 2),
                torch_copy_GBps=round(rate(nb, us_torch), 1), copied=ok,
                note="device copy of %d MiB (read + write bytes), events around %d copies: a flat copy kernel (one "
                     "wave per 1 KiB) and torch's copy_" % (mib, n))


def measure_decode(ep, W, dev, n):
    """The decode shape (128 tokens x 7168, 256 experts, top-8, FP8, alignment 128, no zero padding): layout +
    dispatch as two calls (two launches) and as one (ep_layout_dispatch: one launch), each timed as n back-to-back
    calls between HIP events; and the whole step (layout, dispatch, combine) captured in a HIP graph both ways:
    a graph of 20 consecutive steps, timed over its replays (one replay per step would time the host's replay
    cost, not the GPU)."""
    import torch

    inp = W.make_inputs("decode")
    c = inp["cfg"]
    idx, w, x = inp["topk_idx"].to(dev), inp["topk_weights"].to(dev), inp["x"].to(dev)
    T, K, E, A = c.num_tokens, c.num_topk, c.num_experts, c.expert_alignment
    ws = torch.empty(ep.ep_layout_workspace_bytes(T, K, E, 1, A), dtype=torch.uint8, device=dev)
    lay = dict(num_tokens_per_rank=torch.empty(1, dtype=torch.int32, device=dev),
               num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=dev),
               is_token_in_rank=torch.empty((T, 1), dtype=torch.uint8, device=dev),
               psum_num_recv_tokens_per_expert=torch.empty(E + 1, dtype=torch.int32, device=dev),
               num_invalid_topk=torch.empty(1, dtype=torch.int32, device=dev))
    h0, _ = ep.ep_get_layout(idx, E, 1, 0, A, workspace=ws, outputs=lay)
    dout = ep.alloc_dispatch_outputs(h0, c.hidden, True, device=dev)
    y = W.random_expert_outputs(h0.recv_capacity, c.hidden, seed=99, device=dev)
    out = torch.empty((T, c.hidden), dtype=torch.bfloat16, device=dev)

    def two_calls():
        h, _ = ep.ep_get_layout(idx, E, 1, 0, A, workspace=ws, outputs=lay)
        ep.ep_dispatch(h, x, w, fp8=True, out=dout)
        return h

    def one_call():
        h, _, _ = ep.ep_layout_dispatch(idx, x, E, 1, 0, A, w, fp8=True, out=dout, workspace=ws, outputs=lay)
        return h

    def graph_step(first, reps=20):
        for _ in range(2):
            ep.ep_combine(first(), y, w, out=out)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                ep.ep_combine(first(), y, w, out=out)
        for _ in range(3):
            g.replay()
        nrep = max(1, n // reps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(nrep):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (nrep * reps)

    res = dict(workload="decode: 128 tok x 7168, 256 experts, top-8, FP8, alignment 128, no zero padding",
               layout_then_dispatch_us=round(events_us(two_calls, n), 2),
               layout_dispatch_one_launch_us=round(events_us(one_call, n), 2),
               combine_us=round(events_us(lambda: ep.ep_combine(h0, y, w, out=out), n), 2),
               step_graph_two_launches_us=round(graph_step(two_calls), 2),
               step_graph_one_launch_us=round(graph_step(one_call), 2),
               step_graph_note="per step of a graph of 20 consecutive steps (layout + dispatch, then combine), "
                               "HIP events around its replays")
    h0.free()
    return res


# ---- main ---------------------------------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_get_dispatch_03_amd as ep
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = W.make_inputs(args.workload)
    cfg = inp["cfg"]
    idx = inp["topk_idx"].to(dev)
    w = inp["topk_weights"].to(dev)
    x = inp["x"].to(dev)
    bias = inp["bias"].to(dev) if inp["bias"] is not None else None

    # persistent buffers (allocated once, outside the timed region)
    T, K, E, R = cfg.num_tokens, cfg.num_topk, cfg.num_experts, cfg.num_ranks
    ws = torch.empty(ep.ep_layout_workspace_bytes(T, K, E, R, cfg.expert_alignment), dtype=torch.uint8, device=dev)
    lay_out = dict(num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=dev),
                   num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=dev),
                   is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=dev),
                   psum_num_recv_tokens_per_expert=torch.empty(E // R + 1, dtype=torch.int32, device=dev),
                   num_invalid_topk=torch.empty(1, dtype=torch.int32, device=dev))
    h0, _ = ep.ep_get_layout(idx, E, R, cfg.rank, cfg.expert_alignment, workspace=ws, outputs=lay_out)
    dout = ep.alloc_dispatch_outputs(h0, cfg.hidden, cfg.fp8, device=dev)
    y = W.random_expert_outputs(h0.recv_capacity, cfg.hidden, seed=1234, device=dev)
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device=dev)
    h0.free()

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def step():
        """One pass of the path: the one-call layout + dispatch, then the combine."""
        h, _, _ = ep.ep_layout_dispatch(idx, x, E, R, cfg.rank, cfg.expert_alignment, w, fp8=cfg.fp8,
                                        do_zero_padding=cfg.zero_padding, out=dout, workspace=ws, outputs=lay_out)
        ep.ep_combine(h, y, w, bias, out=out)
        return h

    progress("steps")
    # W untimed warm-up steps
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, bracketed by device syncs
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # the step's own kernels, traced over K more steps (after the timed region, so that it is untouched)
    step_kernels = traced_kernels_us(step, args.steps) if args.trace else {}

    # the same step as a HIP graph: W warm-up replays, then K timed replays
    step_graph_us = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(max(args.warmup, 1)):
            graph.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        step_graph_us = round((time.perf_counter() - g0) * 1e6 / args.steps, 2)
        del graph

    # the same eager step with x taken in turn from 8 copies (470 MB at prefill, more than the 256 MB
    # memory-side cache), so that the dispatch never finds rows an earlier step left in that cache: context for
    # the headline step, which reads the same x every step, as a layer's router leaves its x there just before
    step_x_cold_us = None
    if args.trace:
        progress("steps with x cold")
        xs = [x.clone() for _ in range(8)]

        def step_x(i):
            h, _, _ = ep.ep_layout_dispatch(idx, xs[i % len(xs)], E, R, cfg.rank, cfg.expert_alignment, w,
                                            fp8=cfg.fp8, do_zero_padding=cfg.zero_padding, out=dout, workspace=ws,
                                            outputs=lay_out)
            ep.ep_combine(h, y, w, bias, out=out)
            return h

        for i in range(len(xs)):
            step_x(i)
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for i in range(args.steps):
            step_x(i)
        torch.cuda.synchronize()
        step_x_cold_us = round((time.perf_counter() - c0) * 1e6 / args.steps, 2)
        del xs

    # device counts after the timed loop
    cnt = lay_out["num_tokens_per_expert"].cpu().numpy()
    psum = lay_out["psum_num_recv_tokens_per_expert"].cpu().numpy()
    ntr = lay_out["num_tokens_per_rank"].cpu().numpy()
    El = E // R
    V = int(cnt[cfg.rank * El:(cfg.rank + 1) * El].sum())
    counts = dict(V=V, P=int(psum[-1]) - V, N_send=int(sum(ntr[r] for r in range(R) if r != cfg.rank)))
    bm = bytes_model(cfg, counts)
    step_bytes = bm["layout"] + bm["dispatch"] + bm["combine"]
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # per-call table of every workload (the headline one first)
    probe = Probe(dev) if (args.flushed or args.bound or args.copy_ceiling) else None
    names = [args.workload] + ([n for n in ALL_WORKLOADS if n != args.workload] if args.workloads else [])
    table = {}
    for name in names:
        progress("workload %s" % name)
        table[name] = measure_workload(ep, W, dev, name, args.steps, probe, flushed=args.flushed)
    head = table[args.workload]["calls"]

    dom = "dispatch" if head["dispatch"]["us"] >= head["combine"]["us"] else "combine"
    dom_kernel = {"dispatch": "k_dispatch_fp8", "combine": "k_combine"}[dom]
    achieved = rate(bm[dom], head[dom]["us"])
    roofline = dict(bound="hbm", kernel=dom_kernel, achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=load_traffic(dom_kernel),
                    algorithmic_bytes=bm[dom], avg_launch_us=round(head[dom]["us"], 2),
                    timing="HIP events around %d back-to-back launches on the launch stream" % args.steps)
    if "us_flushed_median" in head[dom]:
        roofline["frac_flushed"] = round(rate(bm[dom], head[dom]["us_flushed_median"]) / HBM_PEAK_GBPS, 4)
    if dom_kernel in step_kernels:
        roofline["in_step_us"] = step_kernels[dom_kernel]
        roofline["frac_in_step"] = round(rate(bm[dom], step_kernels[dom_kernel]) / HBM_PEAK_GBPS, 4)

    progress("dispatch bound, epilogues, decode, copy ceiling")
    bound = None
    combine_bound = None
    if args.bound and args.workload == "prefill":
        bound = measure_dispatch_bound(ep, W, dev, args.steps, probe)
        combine_bound = measure_combine_bound(ep, W, dev, args.steps, probe)
    elif args.bound and args.workload == "ep8":
        bound = measure_send_bound(ep, W, dev, args.steps, probe)
    epi = measure_epilogues(ep, W, dev, args.steps, probe if args.flushed else None) if args.epilogues else None
    decode = measure_decode(ep, W, dev, args.steps) if args.decode else None
    copy_ceiling = measure_copy_ceiling(dev, 20, probe) if args.copy_ceiling else None
    del probe

    cpu = None
    if not args.no_cpu_baseline:
        progress("cpu baseline")
        y_bits = y.cpu().view(torch.int16).numpy().view(np.uint16)
        cpu = cpu_baseline(inp, y_bits, cfg)

    line = dict(
        metric="dispatch/combine effective HBM GB/s + % of peak, 4096 tok×7168 top-8, 1 GPU",
        value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16/fp8-e4m3", data="synthetic",
        config=dict(workload=describe(cfg), tokens=T, hidden=cfg.hidden, experts=E, topk=K, ranks=R,
                    expert_alignment=cfg.expert_alignment, valid_rows=V, pad_rows=counts["P"],
                    A_pad=round(int(psum[-1]) / max(V, 1), 4),
                    data_dtypes="x bf16 -> recv e4m3 + fp32 scales; y bf16 -> out bf16 (fp32 accumulate)"),
        tokens_per_s=round(T / (ms_per_step * 1e-3), 1),
        timing="step: K eager steps of ep_layout_dispatch (the layout kernels, then the dispatch) + "
               "ep_combine between device syncs, host clock; per call: events around K back-to-back launches, "
               "and flushed (2 GiB read sweep before each of 10 + 50 samples, kernel durations from a trace)",
        step_graph_replay_us=step_graph_us,
        step_x_cold_us=step_x_cold_us,
        step_kernels_us=step_kernels,
        kernels=head,
        roofline=roofline,
        cpu_baseline=cpu,
        dispatch_bound=bound,
        combine_bound=combine_bound,
        workloads=table,
        epilogues=epi,
        decode=decode,
        copy_ceiling=copy_ceiling,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
