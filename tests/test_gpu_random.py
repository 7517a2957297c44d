"""Seeded random sweep of shapes through the C ABI against the oracle: for each case a random routing table
(with -1, out-of-range ids and duplicates), random sizes (tokens across tile boundaries, top-k, experts, ranks,
rank, alignment, hidden, BF16 or FP8, zero padding or not, expert- or token-major), then layout, dispatch (both
ep_get_layout + ep_dispatch and the one-call ep_layout_dispatch) and combine, bit for bit against the oracle for
layout and dispatch, within the combine tolerance for combine."""
import numpy as np
import pytest
import torch

import harness as Hn
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
NCASES = 40


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.choice([1, 1, 2, 4, 8, 16]))
    epr = int(rng.integers(1, 1024 // R + 1)) if rng.random() < 0.3 else int(rng.integers(1, 65))
    E = R * epr
    T = int(rng.choice([0, 1, int(rng.integers(2, 256)), 256, int(rng.integers(257, 700))]))
    K = int(rng.integers(1, min(E, 12) + 1)) if rng.random() < 0.8 else int(rng.integers(1, 33))
    fp8 = bool(rng.random() < 0.6)
    H = 128 * int(rng.integers(1, 17)) if fp8 else 8 * int(rng.integers(1, 257))
    A = int(rng.choice([1, 2, 7, 16, 128, int(rng.integers(1, 300))]))
    rank = int(rng.integers(0, R))
    zp = bool(rng.random() < 0.5)
    expand = bool(rng.random() < 0.7)
    idx = rng.integers(0, E, size=(T, K)).astype(np.int64)
    if T > 0 and rng.random() < 0.5:
        m = rng.random((T, K))
        idx[m < 0.1] = -1
        idx[(m >= 0.1) & (m < 0.13)] = E + 3
        idx[(m >= 0.13) & (m < 0.15)] = -7
    gen = torch.Generator().manual_seed(seed)
    w = W.softmax_weights(torch.randn(T, K, generator=gen))
    x = W.normal_bf16((T, H), gen)
    cfg = W.Config("rand%d" % seed, T, H, E, K, "uniform", A, zp, fp8, num_ranks=R, rank=rank)
    return dict(cfg=cfg, topk_idx=torch.from_numpy(idx), topk_weights=w, x=x, bias=None), expand


@pytest.mark.parametrize("seed", range(NCASES))
def test_random_case(seed):
    import combine_get_dispatch_03_amd as ep

    inp, expand = _case(seed)
    c = inp["cfg"]
    print("[random %d] T=%d K=%d E=%d R=%d rank=%d A=%d H=%d fp8=%d zp=%d expand=%d" % (
        seed, c.num_tokens, c.num_topk, c.num_experts, c.num_ranks, c.rank, c.expert_alignment, c.hidden, c.fp8,
        c.zero_padding, expand), flush=True)
    olay, od = Hn.oracle_run(inp, do_expand=expand)
    h, glay, gout = Hn.gpu_layout_dispatch(ep, inp, DEV, do_expand=expand)
    Hn.assert_layout_equal(glay, olay, c)
    Hn.assert_dispatch_equal(gout, od, c)
    # the one-call path on the same inputs
    tmp = ep.Handle(None, torch.empty(0, dtype=torch.int64), None, c.num_tokens, c.num_topk, c.num_experts,
                    c.num_ranks, c.rank, c.expert_alignment)
    out2 = Hn.fill_canaries(ep.alloc_dispatch_outputs(tmp, c.hidden, c.fp8, device=DEV, do_expand=expand))
    h2, glay2, gout2 = ep.ep_layout_dispatch(inp["topk_idx"].to(DEV), inp["x"].to(DEV), c.num_experts, c.num_ranks,
                                             c.rank, c.expert_alignment, inp["topk_weights"].to(DEV), fp8=c.fp8,
                                             do_expand=expand, do_zero_padding=c.zero_padding, out=out2)
    Hn.assert_layout_equal(glay2, olay, c)
    Hn.assert_dispatch_equal(gout2, od, c)
    # combine through the first handle
    T, H = c.num_tokens, c.hidden
    w = inp["topk_weights"]
    if expand:
        y = W.random_expert_outputs(max(h.recv_capacity, 1), H, seed=seed, device=DEV)
        got = ep.ep_combine(h, y, w.to(DEV))
        ref = O.combine(Hn.to_np(y), olay["slot"], w.numpy(), None)
    else:
        y = W.random_expert_outputs(max(T, 1), H, seed=seed, device=DEV)
        got = ep.ep_combine_tokens(h, y)
        ref = O.combine_tokens(Hn.to_np(y), olay["send_slot"], c.rank)
    torch.cuda.synchronize()
    ok, mabs, mrel, nbad = Hn.combine_check(Hn.to_np(got), ref)
    assert ok, (mabs, mrel, nbad)
