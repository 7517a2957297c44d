"""Benchmark of the MoE expert-parallel layout / dispatch / combine path on one MI355X.

A step is one pass of the whole path over one batch of the prefill workload: the layout and the FP8 dispatch
with zero padding (one ep_layout_dispatch call, whose layout kernels also read the token rows ahead of the
dispatch), then the weighted BF16 combine (4096 tokens, hidden 7168, 256 experts in 8 groups with group-limited
top-4-group / top-8 routing, alignment 128).  Inputs and expert outputs are resident in HBM before timing
starts.  W untimed warm-up steps, then exactly K timed steps bracketed by device syncs; the host enqueues the
calls of a step (~35 us of host time) far faster than the GPU runs them (~175 us), so no step waits on the
host.  The same step captured in a HIP graph and replayed K times is reported too
(`step_graph_replay_us`): each replay adds a few microseconds of GPU-side overhead that a graph of a whole
model pass would spread over many more kernels.  Each call's average duration comes from HIP events on the
launch stream around K back-to-back launches of that call, enqueued by the host ahead of the GPU.

Prints one JSON line.  `value` is the step's effective HBM throughput: the algorithmic bytes of layout +
dispatch + combine per step divided by the measured step time.  Algorithmic bytes are what the method must
move: every token row read once, every routed row written once, padding rows when zero padding is requested,
the expert rows gathered once by combine and the output written once (the byte model is in
bytes_model()).  Two extra objects: `roofline` for the dominant kernel and `cpu_baseline` (the oracle timed
on the host).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--flush-samples 50] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill.json")
# the source files each kernel is compiled from (their hash marks counter figures taken from an older kernel)
KERNEL_SOURCES = {
    "k_dispatch_fp8": ("ep_dispatch.hip", "ep_dispatch_core.hpp", "ep_device.hpp"),
    "k_combine": ("ep_combine.hip", "ep_device.hpp"),
    "layout": ("ep_layout.hip", "ep_layout_core.hpp", "ep_device.hpp"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--flush-samples", type=int, default=50,
                    help="per-kernel samples with a cache flush before each (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the steps (counter calibration)")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-epilogues", dest="epilogues", action="store_false",
                    help="skip the receiver-placement / source-reduce measurement at the EP8 shapes")
    ap.add_argument("--no-workloads", dest="workloads", action="store_false",
                    help="skip the per-call summary of the other workloads (tiny, decode, ep8, skewed)")
    ap.add_argument("--no-copy-ceiling", dest="copy_ceiling", action="store_false",
                    help="skip the timed plain device copy reported as context")
    ap.add_argument("--no-decode", dest="decode", action="store_false",
                    help="skip the decode-shape comparison of the one-launch layout + dispatch")
    return ap.parse_args()


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


def cpu_baseline(inp, y_bits, cfg):
    """The oracle as it stands (single thread, plain C) on the full workload, pinned to one host core, repeated
    until about 10 s of CPU time have been spent (at least 3 runs); the median run is reported."""
    import numpy as np

    import oracle as O
    import workloads as W

    idx = inp["topk_idx"].numpy()
    w = inp["topk_weights"].numpy()
    x = W.bf16_bits(inp["x"])
    bias = W.bf16_bits(inp["bias"]) if inp["bias"] is not None else None
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})
    times = []
    while len(times) < 3 or sum(times) < 10.0:
        t0 = time.perf_counter()
        lay = O.layout(idx, cfg.num_experts, cfg.num_ranks, cfg.rank, cfg.expert_alignment)
        O.dispatch(x, idx, w, lay, cfg.num_experts, cfg.num_ranks, cfg.rank, cfg.expert_alignment, fp8=cfg.fp8,
                   zero_pad=cfg.zero_padding, recv_fill=None)
        O.combine(y_bits, lay["slot"], w, bias)
        times.append(time.perf_counter() - t0)
    os.sched_setaffinity(0, set(allowed))
    El = cfg.num_experts // cfg.num_ranks
    cnt = lay["cnt"][cfg.rank * El:(cfg.rank + 1) * El]
    V = int(cnt.sum())
    counts = dict(V=V, P=int(lay["psum"][-1]) - V, N_send=int(sum(lay["ntok_rank"][r] for r in range(cfg.num_ranks)
                                                                    if r != cfg.rank)))
    bm = bytes_model(cfg, counts)
    total = bm["layout"] + bm["dispatch"] + bm["combine"]
    med = float(np.median(times))
    return dict(value=round(total / med / 1e9, 3), unit="GB/s", cores=1, kind="oracle",
                sample="full %s workload (layout + FP8 dispatch + combine), median of %d runs, %.2f s each"
                       % (cfg.name, len(times), med),
                pinned_core=core, host_cores_available=len(allowed), host_cpu=host_cpu_model())


def measure_epilogues(ep, W, dev, n):
    """Receiver-side placement and source-side reduce at the EP8 shapes: rank 0 (experts 0..31 of 256) receiving
    the rows of 7 other ranks of 4096 tokens each (top-8 uniform routing, FP8 rows + 56 scales, alignment 128),
    and the reduce of 8 returned windows of 4096 x 7168 BF16 rows with the local part and a bias."""
    import numpy as np
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

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.02))
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    t_rows = timed(lambda: ep.ep_dispatch_rows(hr, rows, sc, tw, do_zero_padding=False, out=out))
    b_rows = n_valid * row_b + R * T * K * 12 + V * (row_b + 8) + P * 8

    inp = W.make_inputs("ep8")
    h0, l0 = ep.ep_get_layout(inp["topk_idx"].to(dev), E, R, 0, A)
    parts = W.random_expert_outputs(R * T, H, seed=3, device=dev).view(R, T, H)
    local = W.random_expert_outputs(T, H, seed=4, device=dev)
    bias = W.random_expert_outputs(T, H, seed=5, device=dev)
    red = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    t_red = timed(lambda: ep.ep_combine_reduce(h0, parts, local, bias, out=red))
    ntr = l0["num_tokens_per_rank"].cpu().numpy()
    n_part = int(sum(ntr[r] for r in range(1, R)))
    b_red = n_part * 2 * H + 3 * T * 2 * H + T * R * 4
    return dict(
        dispatch_rows=dict(us=round(t_rows * 1e3, 2), bytes=b_rows, GBps=round(b_rows / (t_rows * 1e-3) / 1e9, 1),
                           received_rows=n_valid, placed_rows=V),
        combine_reduce=dict(us=round(t_red * 1e3, 2), bytes=b_red, GBps=round(b_red / (t_red * 1e-3) / 1e9, 1),
                            partial_rows=n_part))


def measure_copy_ceiling(dev, n, mib=1024):
    """A plain device-to-device copy of `mib` MiB (torch's copy_, the runtime's copy kernel), timed with events
    over n back-to-back copies: the streaming rate this GPU reaches on a flat read + flat write, as context for
    the kernels' rates (not the roofline's denominator, which is the published 8 TB/s)."""
    import torch

    a = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    del a, b
    return dict(bytes_per_copy=2 * (mib << 20), us=round(us, 2), GBps=round(2 * (mib << 20) / (us * 1e-6) / 1e9, 1),
                note="device copy of %d MiB (read + write bytes), events around %d copies" % (mib, n))


def measure_workloads(ep, W, dev, names, n):
    """The other workloads at a glance, measured like the headline one: per call, HIP events around n back-to-back
    launches; the step (one-call layout + dispatch, then combine), the median of five blocks of n eager steps
    between device syncs, host clock; algorithmic bytes from the byte model with the device counts.  Parity for
    each is in the test suite."""
    import time

    import numpy as np
    import torch

    out = {}
    for name in names:
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

        def timed(fn):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(int(2.4e9 * 0.02))
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n

        def step():
            hs, _, _ = ep.ep_layout_dispatch(idx, x, E, R, cfg.rank, A, w, fp8=cfg.fp8,
                                             do_zero_padding=cfg.zero_padding, out=dout, workspace=ws, outputs=lay)
            ep.ep_combine(hs, y, w, bias, out=res)

        us = dict(layout=timed(lambda: ep.ep_get_layout(idx, E, R, cfg.rank, A, workspace=ws, outputs=lay)),
                  dispatch=timed(lambda: ep.ep_dispatch(h, x, w, fp8=cfg.fp8, do_zero_padding=cfg.zero_padding,
                                                        out=dout)),
                  combine=timed(lambda: ep.ep_combine(h, y, w, bias, out=res)))
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        # five blocks of n steps between device syncs, host clock; the median block, so that one stall of the
        # host (these steps are short, and for tiny and decode bound by the host's enqueue) does not set it
        blocks = []
        for _ in range(5):
            t0 = time.perf_counter()
            for _ in range(n):
                step()
            torch.cuda.synchronize()
            blocks.append((time.perf_counter() - t0) * 1e6 / n)
        step_us = float(np.median(blocks))
        cnt = lay["num_tokens_per_expert"].cpu().numpy()
        psum = lay["psum_num_recv_tokens_per_expert"].cpu().numpy()
        ntr = lay["num_tokens_per_rank"].cpu().numpy()
        El = E // R
        V = int(cnt[cfg.rank * El:(cfg.rank + 1) * El].sum())
        bm = bytes_model(cfg, dict(V=V, P=int(psum[-1]) - V,
                                   N_send=int(sum(ntr[r] for r in range(R) if r != cfg.rank))))
        rate = lambda b, u: b / (u * 1e-6) / 1e9
        out[name] = dict(
            layout_us=round(us["layout"], 2), dispatch_us=round(us["dispatch"], 2),
            dispatch_GBps=round(rate(bm["dispatch"], us["dispatch"]), 1),
            dispatch_pct_peak=round(100 * rate(bm["dispatch"], us["dispatch"]) / HBM_PEAK_GBPS, 1),
            combine_us=round(us["combine"], 2), combine_GBps=round(rate(bm["combine"], us["combine"]), 1),
            combine_pct_peak=round(100 * rate(bm["combine"], us["combine"]) / HBM_PEAK_GBPS, 1),
            step_us=round(step_us, 2),
            step_GBps=round(rate(bm["layout"] + bm["dispatch"] + bm["combine"], step_us), 1))
        h.free()
        del ws, lay, dout, y, res, idx, w, x, bias
        torch.cuda.empty_cache()
    return out


def measure_decode(ep, W, dev, n):
    """The decode shape (128 tokens x 7168, 256 experts, top-8, FP8, alignment 128, no zero padding): layout +
    dispatch as two calls (ep_get_layout, ep_dispatch: two launches) and as one (ep_layout_dispatch: one
    launch), each timed as n back-to-back calls between HIP events; and the whole step (layout, dispatch,
    combine) captured in a HIP graph both ways, timed over n replays."""
    import time

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

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.02))
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def graph_step(first, reps=20):
        # reps consecutive decode steps captured in one graph, so that the host's cost of a replay is spread over
        # them; HIP events around the replays give the GPU-side time of a step
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
               layout_then_dispatch_us=round(timed(two_calls), 2),
               layout_dispatch_one_launch_us=round(timed(one_call), 2),
               combine_us=round(timed(lambda: ep.ep_combine(h0, y, w, out=out)), 2),
               step_graph_two_launches_us=round(graph_step(two_calls), 2),
               step_graph_one_launch_us=round(graph_step(one_call), 2),
               step_graph_note="per step of a graph of 20 consecutive steps (layout + dispatch, then combine), "
                               "HIP events around its replays")
    h0.free()
    return res


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

    def step(ev=None):
        """One pass of the path.  Timed steps (ev None) make the one-call layout + dispatch, which reads the token
        rows into the memory-side cache while the layout runs; the flushed per-call samples (ev given) make the
        two calls separately so that each can be bracketed by its own events."""
        stream = torch.cuda.current_stream()
        if ev is None:
            h, _, _ = ep.ep_layout_dispatch(idx, x, E, R, cfg.rank, cfg.expert_alignment, w, fp8=cfg.fp8,
                                            do_zero_padding=cfg.zero_padding, out=dout, workspace=ws,
                                            outputs=lay_out)
            ep.ep_combine(h, y, w, bias, out=out)
            return h
        ev[0].record(stream)
        h, _ = ep.ep_get_layout(idx, E, R, cfg.rank, cfg.expert_alignment, workspace=ws, outputs=lay_out)
        ev[1].record(stream)
        ep.ep_dispatch(h, x, w, fp8=cfg.fp8, do_zero_padding=cfg.zero_padding, out=dout)
        ev[2].record(stream)
        ep.ep_combine(h, y, w, bias, out=out)
        ev[3].record(stream)
        return h

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

    # the same step as a HIP graph: W warm-up replays, then K timed replays
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graph_handle = step()
    torch.cuda.synchronize()
    for _ in range(max(args.warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    g0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    step_graph_us = (time.perf_counter() - g0) * 1e6 / args.steps

    # per-kernel durations: HIP events on the launch stream bracketing N back-to-back launches of one call
    # (an event marker between kernels costs several microseconds of GPU time, so each kernel is timed in a run
    # of its own launches and the marker cost is divided by N); the calls are the same as inside the step
    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.02))   # ~20 ms of GPU spin while the host enqueues the launches
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    hk, _ = ep.ep_get_layout(idx, E, R, cfg.rank, cfg.expert_alignment, workspace=ws, outputs=lay_out)
    avg = {
        "layout": timed(lambda: ep.ep_get_layout(idx, E, R, cfg.rank, cfg.expert_alignment, workspace=ws,
                                                 outputs=lay_out), args.steps),
        "dispatch": timed(lambda: ep.ep_dispatch(hk, x, w, fp8=cfg.fp8, do_zero_padding=cfg.zero_padding,
                                                 out=dout), args.steps),
        "combine": timed(lambda: ep.ep_combine(hk, y, w, bias, out=out), args.steps),
    }

    def layout_then_dispatch():
        h, _ = ep.ep_get_layout(idx, E, R, cfg.rank, cfg.expert_alignment, workspace=ws, outputs=lay_out)
        ep.ep_dispatch(h, x, w, fp8=cfg.fp8, do_zero_padding=cfg.zero_padding, out=dout)

    layout_dispatch_us = timed(layout_then_dispatch, args.steps) * 1e3

    def layout_dispatch_one_call():
        ep.ep_layout_dispatch(idx, x, E, R, cfg.rank, cfg.expert_alignment, w, fp8=cfg.fp8,
                              do_zero_padding=cfg.zero_padding, out=dout, workspace=ws, outputs=lay_out)

    layout_dispatch_one_us = timed(layout_dispatch_one_call, args.steps) * 1e3

    # per-kernel samples with a cache flush before each (10 warm-up + N samples, the pages' method)
    flushed = None
    if args.flush_samples > 0:
        junk = torch.empty(2 << 30, dtype=torch.uint8, device=dev).fill_(3)
        fl = {"layout": [], "dispatch": [], "combine": []}
        for i in range(10 + args.flush_samples):
            junk.sum(dtype=torch.int64)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            step(ev)
            torch.cuda.synchronize()
            if i >= 10:
                fl["layout"].append(ev[0].elapsed_time(ev[1]))  # includes event-marker overhead
                fl["dispatch"].append(ev[1].elapsed_time(ev[2]))
                fl["combine"].append(ev[2].elapsed_time(ev[3]))
        del junk
        flushed = {k: float(np.median(v)) for k, v in fl.items()}
        flushed_min = {k: float(np.min(v)) for k, v in fl.items()}

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

    def gbps(b, ms):
        return b / (ms * 1e-3) / 1e9

    kern = {
        "layout": dict(us=round(avg["layout"] * 1e3, 2), bytes=bm["layout"]),
        "dispatch": dict(us=round(avg["dispatch"] * 1e3, 2), bytes=bm["dispatch"],
                         GBps=round(gbps(bm["dispatch"], avg["dispatch"]), 1),
                         pct_peak=round(100 * gbps(bm["dispatch"], avg["dispatch"]) / HBM_PEAK_GBPS, 1)),
        "combine": dict(us=round(avg["combine"] * 1e3, 2), bytes=bm["combine"],
                        GBps=round(gbps(bm["combine"], avg["combine"]), 1),
                        pct_peak=round(100 * gbps(bm["combine"], avg["combine"]) / HBM_PEAK_GBPS, 1)),
    }
    if flushed is not None:
        for k in ("dispatch", "combine"):
            kern[k]["us_flushed_median"] = round(flushed[k] * 1e3, 2)
            kern[k]["us_flushed_min"] = round(flushed_min[k] * 1e3, 2)
            kern[k]["GBps_flushed"] = round(gbps(bm[k], flushed[k]), 1)
        kern["layout"]["us_flushed_median"] = round(flushed["layout"] * 1e3, 2)
        kern["layout"]["us_flushed_min"] = round(flushed_min["layout"] * 1e3, 2)
    kern["layout_then_dispatch"] = dict(us=round(layout_dispatch_us, 2))
    kern["layout_dispatch_one_call"] = dict(us=round(layout_dispatch_one_us, 2),
                                            note="ep_layout_dispatch: the layout kernels also read x ahead of "
                                                 "the dispatch")

    dom = "dispatch" if avg["dispatch"] >= avg["combine"] else "combine"
    dom_kernel = {"dispatch": "k_dispatch_fp8", "combine": "k_combine"}[dom]
    achieved = gbps(bm[dom], avg[dom])
    roofline = dict(bound="hbm", kernel=dom_kernel, achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=load_traffic(dom_kernel),
                    algorithmic_bytes=bm[dom], avg_launch_us=round(avg[dom] * 1e3, 2))

    epi = measure_epilogues(ep, W, dev, args.steps) if args.epilogues else None
    decode = measure_decode(ep, W, dev, args.steps) if args.decode else None
    copy_ceiling = measure_copy_ceiling(dev, 20) if args.copy_ceiling else None
    others = ([n for n in ("tiny", "decode", "ep8", "skewed") if n != args.workload] if args.workloads else [])
    workloads = measure_workloads(ep, W, dev, others, 20) if others else None
    if workloads:
        workloads["note"] = ("per call: events around back-to-back launches; step: eager one-call layout + dispatch "
                             "then combine, host clock, the median of five blocks of 20 steps -- for tiny and decode "
                             "that is bounded by the host's enqueue of the calls, see decode.step_graph_* for the "
                             "GPU-side decode step")

    cpu = None
    if not args.no_cpu_baseline:
        y_bits = y.cpu().view(torch.int16).numpy().view(np.uint16)
        cpu = cpu_baseline(inp, y_bits, cfg)

    line = dict(
        metric="dispatch/combine effective HBM GB/s + % of peak, 4096 tok\u00d77168 top-8, 1 GPU",
        value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16/fp8-e4m3", data="synthetic",
        config=dict(workload="%s: %d tok x hidden %d, %d experts%s, top-%d, FP8 e4m3 per-128 dispatch%s, "
                              "BF16 combine, alignment %d" % (
                                  cfg.name, T, cfg.hidden, E,
                                  " (8 groups, top-4 groups)" if cfg.routing == "grouped" else "", K,
                                  " + zero padding" if cfg.zero_padding else "", cfg.expert_alignment),
                    tokens=T, hidden=cfg.hidden, experts=E, topk=K, ranks=R, expert_alignment=cfg.expert_alignment,
                    valid_rows=V, pad_rows=counts["P"], A_pad=round(int(psum[-1]) / max(V, 1), 4),
                    data_dtypes="x bf16 -> recv e4m3 + fp32 scales; y bf16 -> out bf16 (fp32 accumulate)"),
        tokens_per_s=round(T / (ms_per_step * 1e-3), 1),
        timing="step: K eager steps of ep_layout_dispatch (layout kernels reading x ahead, then the dispatch) + "
               "ep_combine between device syncs; per call: "
               "events around K back-to-back launches",
        step_graph_replay_us=round(step_graph_us, 2),
        kernels=kern,
        roofline=roofline,
        cpu_baseline=cpu,
        epilogues=epi,
        decode=decode,
        copy_ceiling=copy_ceiling,
        workloads=workloads,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
