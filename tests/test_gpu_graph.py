"""The whole path is capturable into a HIP graph: no call synchronises, allocates or copies to the host.
The decode-shaped workload (layout -> FP8 dispatch -> combine, as three calls or as the one-launch
ep_layout_dispatch + combine) is captured once and replayed several times, with eager work between replays
(canary refills of every output, a new x between replays); every replay must equal the eager results bit for
bit."""
import numpy as np
import pytest
import torch

import harness as Hn
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _fill_canary(t):
    if t is None:
        return
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(-23131)
    elif t.dtype == torch.uint8:
        t.fill_(0xA5)
    elif t.dtype == torch.float32:
        t.fill_(-7.0)
    else:
        t.fill_(-7)


@pytest.mark.parametrize("name,fused", [("decode", False), ("tiny", False), ("decode", True), ("tiny", True)])
def test_graph_capture_and_replay(name, fused):
    import combine_get_dispatch_03_amd as ep

    inp = W.make_inputs(name)
    c = inp["cfg"]
    T, K, E, R, A = c.num_tokens, c.num_topk, c.num_experts, c.num_ranks, c.expert_alignment
    idx = inp["topk_idx"].to(DEV)
    w = inp["topk_weights"].to(DEV)
    x = inp["x"].to(DEV).clone()
    x2 = W.normal_bf16((T, c.hidden), torch.Generator().manual_seed(123)).to(DEV)
    ws = torch.empty(ep.ep_layout_workspace_bytes(T, K, E, R, A), dtype=torch.uint8, device=DEV)
    lay = dict(num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=DEV),
               num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=DEV),
               is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=DEV),
               psum_num_recv_tokens_per_expert=torch.empty(E // R + 1, dtype=torch.int32, device=DEV),
               num_invalid_topk=torch.empty(1, dtype=torch.int32, device=DEV))
    cap = ep.ep_recv_capacity(T, K, E // R, A)
    h0, _ = ep.ep_get_layout(idx, E, R, 0, A, workspace=ws, outputs=lay)
    dout = ep.alloc_dispatch_outputs(h0, c.hidden, c.fp8, device=DEV)
    y = W.random_expert_outputs(cap, c.hidden, seed=9, device=DEV)
    out = torch.empty((T, c.hidden), dtype=torch.bfloat16, device=DEV)

    def refill():
        for t in list(lay.values()) + list(dout.values()) + [out]:
            _fill_canary(t)

    def run():
        if fused:
            h, _, _ = ep.ep_layout_dispatch(idx, x, E, R, 0, A, w, fp8=c.fp8, do_zero_padding=c.zero_padding,
                                            out=dout, workspace=ws, outputs=lay)
        else:
            h, _ = ep.ep_get_layout(idx, E, R, 0, A, workspace=ws, outputs=lay)
            ep.ep_dispatch(h, x, w, fp8=c.fp8, do_zero_padding=c.zero_padding, out=dout)
        ep.ep_combine(h, y, w, None, out=out)
        return h

    def snapshot():
        torch.cuda.synchronize()
        return [Hn.to_np(t) for t in list(lay.values()) + [v for v in dout.values() if v is not None] + [out]]

    # eager references for x and x2
    refill()
    run()
    ref1 = snapshot()
    x_saved = x.clone()
    x.copy_(x2)
    refill()
    run()
    ref2 = snapshot()
    x.copy_(x_saved)

    g = torch.cuda.CUDAGraph()
    refill()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        hg = run()
    torch.cuda.synchronize()

    for r, use_x2 in enumerate([False, True, False, True]):
        x.copy_(x2 if use_x2 else x_saved)       # eager work between replays
        refill()
        g.replay()
        got = snapshot()
        ref = ref2 if use_x2 else ref1
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), "replay %d differs from the eager result" % r
    del hg
