"""Streams: every call enqueues its kernels on the stream it is given (`stream=`) or, without one, on torch's
current stream.  The calls are captured in a HIP graph on a side stream -- either passed explicitly while
torch's current stream is another one, or taken from the current stream -- and only work enqueued on the
capturing stream lands in the graph.  The outputs are then reset to canaries and the graph is replayed: every
output must come back equal, bit for bit, to the same calls made eagerly on the default stream (the kernels are
deterministic), so a kernel enqueued anywhere else would leave canaries behind."""
import pytest
import torch

import harness as Hn
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ep():
    import combine_get_dispatch_03_amd as ep
    return ep


def _buffers(ep, c, cap):
    """Every output and the workspace, allocated up front (nothing is allocated during a capture)."""
    T, E, R = c.num_tokens, c.num_experts, c.num_ranks
    tmp = ep.Handle(None, None, None, T, c.num_topk, E, R, c.rank, c.expert_alignment)
    return dict(
        ws=torch.empty(ep.ep_layout_workspace_bytes(T, c.num_topk, E, R, c.expert_alignment), dtype=torch.uint8,
                       device=DEV),
        lay=dict(num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=DEV),
                 num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=DEV),
                 is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=DEV),
                 psum_num_recv_tokens_per_expert=torch.empty(E // R + 1, dtype=torch.int32, device=DEV),
                 num_invalid_topk=torch.empty(1, dtype=torch.int32, device=DEV)),
        out=ep.alloc_dispatch_outputs(tmp, c.hidden, c.fp8, device=DEV),
        res=torch.empty((T, c.hidden), dtype=torch.bfloat16, device=DEV))


def _reset(b):
    Hn.fill_canaries(b["out"])
    for t in b["lay"].values():
        t.fill_(0x5A)
    b["res"].view(torch.int16).fill_(0x7F7F)


def _path(ep, c, idx, x, w, y, b, two_calls, stream):
    """layout + dispatch (one call, or ep_get_layout then ep_dispatch) and combine; every call gets `stream`."""
    if two_calls:
        h, _ = ep.ep_get_layout(idx, c.num_experts, c.num_ranks, c.rank, c.expert_alignment, workspace=b["ws"],
                                outputs=b["lay"], stream=stream)
        ep.ep_dispatch(h, x, w, fp8=c.fp8, do_zero_padding=c.zero_padding, out=b["out"], stream=stream)
    else:
        h, _, _ = ep.ep_layout_dispatch(idx, x, c.num_experts, c.num_ranks, c.rank, c.expert_alignment, w,
                                        fp8=c.fp8, do_zero_padding=c.zero_padding, out=b["out"], workspace=b["ws"],
                                        outputs=b["lay"], stream=stream)
    ep.ep_combine(h, y, w, out=b["res"], stream=stream)
    return h


def _assert_same(a, b):
    for k, t in a["lay"].items():
        assert torch.equal(t, b["lay"][k]), k
    for k, t in a["out"].items():
        if t is not None:
            assert torch.equal(t.view(torch.uint8), b["out"][k].view(torch.uint8)), k
    assert torch.equal(a["res"].view(torch.int16), b["res"].view(torch.int16))


@pytest.mark.parametrize("name", ["decode", "prefill"])
@pytest.mark.parametrize("two_calls", [False, True])
@pytest.mark.parametrize("how", ["current", "explicit"])
def test_calls_follow_stream(ep, name, two_calls, how):
    inp = W.make_inputs(name)
    c = inp["cfg"]
    print("[streams] %s two_calls=%d %s" % (name, two_calls, how), flush=True)
    idx, w, x = inp["topk_idx"].to(DEV), inp["topk_weights"].to(DEV), inp["x"].to(DEV)
    cap = ep.ep_recv_capacity(c.num_tokens, c.num_topk, c.num_experts // c.num_ranks, c.expert_alignment)
    y = W.random_expert_outputs(cap, c.hidden, seed=5, device=DEV)

    ref = _buffers(ep, c, cap)
    _reset(ref)
    _path(ep, c, idx, x, w, y, ref, two_calls, None).free()
    torch.cuda.synchronize()

    got = _buffers(ep, c, cap)
    _reset(got)
    torch.cuda.synchronize()
    side, other = torch.cuda.Stream(), torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        if how == "current":
            h = _path(ep, c, idx, x, w, y, got, two_calls, None)
        else:
            with torch.cuda.stream(other):     # torch's current stream is not the one passed
                h = _path(ep, c, idx, x, w, y, got, two_calls, side)
    torch.cuda.synchronize()
    _reset(got)                                # whatever ran outside the graph is wiped
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    _assert_same(ref, got)
    h.free()


def test_threads_call_concurrently(ep):
    """Two host threads run the path at the same time, each on its own stream with its own inputs and buffers
    (the binding releases the GIL inside every library call, so the calls overlap in the library).  Each
    thread's outputs equal those of the same calls made alone: the library keeps no shared per-call state."""
    import threading
    cases = []
    for name, seed in (("decode", 3), ("prefill", 4)):
        inp = W.make_inputs(name, seed=seed)
        c = inp["cfg"]
        cap = ep.ep_recv_capacity(c.num_tokens, c.num_topk, c.num_experts // c.num_ranks, c.expert_alignment)
        cases.append(dict(c=c, idx=inp["topk_idx"].to(DEV), w=inp["topk_weights"].to(DEV), x=inp["x"].to(DEV),
                          y=W.random_expert_outputs(cap, c.hidden, seed=seed, device=DEV), cap=cap))
    refs = []
    for k in cases:
        b = _buffers(ep, k["c"], k["cap"])
        _reset(b)
        _path(ep, k["c"], k["idx"], k["x"], k["w"], k["y"], b, False, None).free()
        torch.cuda.synchronize()
        refs.append(b)

    errors = []
    def worker(i, k):
        # Everything a thread allocates, writes and compares stays on its own stream.  (Buffers taken from the
        # default stream's pool, which both threads share, and written on a side stream could be handed out while
        # the other thread's default-stream work on them is still queued: torch's caching allocator orders a
        # freed block only after the work of its own stream.)
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for rep in range(20):
                    b = _buffers(ep, k["c"], k["cap"])
                    _reset(b)
                    _path(ep, k["c"], k["idx"], k["x"], k["w"], k["y"], b, rep % 2 == 1, None).free()
                    s.synchronize()
                    _assert_same(refs[i], b)
                    s.synchronize()
        except Exception as exc:   # reported by the main thread
            errors.append((i, repr(exc)))

    threads = [threading.Thread(target=worker, args=(i, k)) for i, k in enumerate(cases)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_binding_allocates_on_given_stream(ep, name):
    """With stream= given and no output tensors, the binding allocates the outputs and workspace itself (with
    the given stream current) while torch's current stream stays the default one; the results on that stream
    equal the default-stream calls bit for bit (rows a call leaves unwritten are compared through the layout
    only: the allocated buffers start uninitialised)."""
    inp = W.make_inputs(name)
    c = inp["cfg"]
    idx, w, x = inp["topk_idx"].to(DEV), inp["topk_weights"].to(DEV), inp["x"].to(DEV)
    cap = ep.ep_recv_capacity(c.num_tokens, c.num_topk, c.num_experts // c.num_ranks, c.expert_alignment)
    y = W.random_expert_outputs(cap, c.hidden, seed=9, device=DEV)
    h0, lay0, out0 = ep.ep_layout_dispatch(idx, x, c.num_experts, c.num_ranks, c.rank, c.expert_alignment, w,
                                           fp8=c.fp8, do_zero_padding=c.zero_padding)
    res0 = ep.ep_combine(h0, y, w)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for _ in range(3):
        h1, lay1, out1 = ep.ep_layout_dispatch(idx, x, c.num_experts, c.num_ranks, c.rank, c.expert_alignment, w,
                                               fp8=c.fp8, do_zero_padding=c.zero_padding, stream=s)
        res1 = ep.ep_combine(h1, y, w, stream=s)
        s.synchronize()
        for k, t in lay0.items():
            assert torch.equal(t, lay1[k]), k
        assert torch.equal(res0.view(torch.int16), res1.view(torch.int16))
        # the written rows: every valid row (recv_src_idx >= 0) and, with zero padding, every row up to psum[-1]
        rows = int(lay0["psum_num_recv_tokens_per_expert"][-1])
        src0, src1 = out0["recv_src_idx"][:rows], out1["recv_src_idx"][:rows]
        assert torch.equal(src0, src1)
        keep = src0 >= 0 if not c.zero_padding else torch.ones_like(src0, dtype=torch.bool)
        assert torch.equal(out0["recv_x"][:rows][keep], out1["recv_x"][:rows][keep])
        h1.free()
    h0.free()
