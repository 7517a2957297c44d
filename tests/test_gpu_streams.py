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
