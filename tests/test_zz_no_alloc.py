"""ep_layout_dispatch_noalloc (the entry point for callers that cannot allocate) against ep_layout_dispatch:
same inputs, every output bit for bit (canary-filled buffers, so untouched rows are compared too), and the
combine through each handle.  Calls run back to back with shrinking inputs, so that a result left in the static
scratch by a larger call would show up in a smaller one: 4096-token prefill (multi-tile layout), the 4096-token
ep8 shape (send windows), 1000 tokens of the prefill routing, then the 128-token decode shape (one-launch path)."""
import numpy as np
import pytest
import torch

import harness as Hn
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
LAYOUT_KEYS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
               "psum_num_recv_tokens_per_expert", "num_invalid_topk")


@pytest.fixture(scope="module")
def ep():
    import combine_get_dispatch_03_amd as ep
    return ep


def _layout_outputs(T, E, R):
    El = E // R
    o = dict(num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=DEV),
             num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=DEV),
             is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=DEV),
             psum_num_recv_tokens_per_expert=torch.empty(El + 1, dtype=torch.int32, device=DEV),
             num_invalid_topk=torch.empty(1, dtype=torch.int32, device=DEV))
    return Hn.fill_canaries(o)


def _subset(inp, n):
    c = inp["cfg"]
    cfg = W.Config(c.name + "_%d" % n, n, c.hidden, c.num_experts, c.num_topk, c.routing, c.expert_alignment,
                   c.zero_padding, c.fp8, num_ranks=c.num_ranks, rank=c.rank)
    return dict(cfg=cfg, topk_idx=inp["topk_idx"][:n].contiguous(), topk_weights=inp["topk_weights"][:n].contiguous(),
                x=inp["x"][:n].contiguous(), bias=None)


def _check_same(ep, inp):
    c = inp["cfg"]
    T, K, E, R, A = c.num_tokens, c.num_topk, c.num_experts, c.num_ranks, c.expert_alignment
    print("[noalloc] %s: T=%d K=%d E=%d R=%d A=%d" % (c.name, T, K, E, R, A), flush=True)
    idx, x, w = inp["topk_idx"].to(DEV), inp["x"].to(DEV), inp["topk_weights"].to(DEV)
    h_ref, _ = ep.ep_get_layout(idx, E, R, c.rank, A)          # only to size the outputs
    out_ref = Hn.dispatch_outputs_with_canary(ep, h_ref, c.hidden, c.fp8, DEV)
    out_new = Hn.dispatch_outputs_with_canary(ep, h_ref, c.hidden, c.fp8, DEV)
    lay_ref, lay_new = _layout_outputs(T, E, R), _layout_outputs(T, E, R)
    h1, _, _ = ep.ep_layout_dispatch(idx, x, E, R, c.rank, A, w, fp8=c.fp8, do_zero_padding=c.zero_padding,
                                     out=out_ref, outputs=lay_ref)
    h2, _, _ = ep.ep_layout_dispatch_noalloc(idx, x, E, out_new, R, c.rank, A, w, fp8=c.fp8,
                                             do_zero_padding=c.zero_padding, outputs=lay_new)
    torch.cuda.synchronize()
    for k in LAYOUT_KEYS:
        assert torch.equal(lay_ref[k], lay_new[k]), k
    for k, t in out_ref.items():
        if t is None:
            assert out_new[k] is None
            continue
        a, b = Hn.to_np(t), Hn.to_np(out_new[k])
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (k, Hn._first_diff(a, b))
    y = W.random_expert_outputs(h1.recv_capacity, c.hidden, seed=T, device=DEV)
    bias = W.normal_bf16((T, c.hidden), torch.Generator().manual_seed(T), 0.1).to(DEV)
    o1 = ep.ep_combine(h1, y, w, bias)
    o2 = ep.ep_combine(h2, y, w, bias)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    h1.free()
    h_ref.free()
    return h2


def test_noalloc_matches_layout_dispatch_shrinking_inputs(ep):
    prefill = W.make_inputs("prefill")
    handles = []
    for inp in (prefill, W.make_inputs("ep8"), _subset(prefill, 1000), W.make_inputs("decode")):
        handles.append(_check_same(ep, inp))
    # one static handle per GPU: every call returned the same object, now holding the last call's layout
    assert len({h.ptr.value for h in handles}) == 1
    assert ep._lib.ep_handle_free(handles[0].ptr) == 0          # freeing it is a no-op ...
    d = W.make_inputs("decode")
    _check_same(ep, d)                                          # ... and it keeps working


def test_noalloc_bf16_token_major(ep):
    """BF16 rows (the copy kernel) and the token-major mode, after the FP8 calls above."""
    inp = W.make_inputs("tiny")
    c = inp["cfg"]
    idx, x, w = inp["topk_idx"].to(DEV), inp["x"].to(DEV), inp["topk_weights"].to(DEV)
    h_ref, _ = ep.ep_get_layout(idx, c.num_experts, 1, 0, c.expert_alignment)
    for expand in (True, False):
        out_ref = Hn.dispatch_outputs_with_canary(ep, h_ref, c.hidden, False, DEV, do_expand=expand)
        out_new = Hn.dispatch_outputs_with_canary(ep, h_ref, c.hidden, False, DEV, do_expand=expand)
        ep.ep_layout_dispatch(idx, x, c.num_experts, 1, 0, c.expert_alignment, w, fp8=False, do_expand=expand,
                              do_zero_padding=True, out=out_ref)
        ep.ep_layout_dispatch_noalloc(idx, x, c.num_experts, out_new, 1, 0, c.expert_alignment, w, fp8=False,
                                      do_expand=expand, do_zero_padding=True)
        torch.cuda.synchronize()
        for k, t in out_ref.items():
            if t is not None:
                assert np.array_equal(Hn.to_np(t).view(np.uint8), Hn.to_np(out_new[k]).view(np.uint8)), (expand, k)


def test_noalloc_in_graph_capture(ep):
    """Its callers' use: captured in a HIP graph.  One eager call first (the per-device set-up), then the call and
    a combine captured, the graph replayed three times with eager work in between (the outputs reset to canaries);
    every replay's outputs equal the eager ones bit for bit."""
    inp = W.make_inputs("decode")
    c = inp["cfg"]
    T, E, A, H = c.num_tokens, c.num_experts, c.expert_alignment, c.hidden
    idx, x, w = inp["topk_idx"].to(DEV), inp["x"].to(DEV), inp["topk_weights"].to(DEV)
    h_ref, _ = ep.ep_get_layout(idx, E, 1, 0, A)                 # only to size the outputs
    out = Hn.dispatch_outputs_with_canary(ep, h_ref, H, True, DEV)
    lay = _layout_outputs(T, E, 1)
    y = W.random_expert_outputs(h_ref.recv_capacity, H, seed=21, device=DEV)
    res = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    h, _, _ = ep.ep_layout_dispatch_noalloc(idx, x, E, out, 1, 0, A, w, fp8=True, outputs=lay)
    ep.ep_combine(h, y, w, out=res)
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in list(out.items()) + list(lay.items()) if t is not None}
    ref["res"] = res.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hg, _, _ = ep.ep_layout_dispatch_noalloc(idx, x, E, out, 1, 0, A, w, fp8=True, outputs=lay)
        ep.ep_combine(hg, y, w, out=res)
    for rep in range(3):
        Hn.fill_canaries(out)
        Hn.fill_canaries(lay)
        res.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dict(list(out.items()) + list(lay.items()), res=res)
        for k, t in ref.items():
            assert torch.equal(got[k].view(torch.uint8), t.view(torch.uint8)), (rep, k)
        Hn.assert_guards(out)
    h_ref.free()
