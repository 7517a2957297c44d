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
    R = int(rng.choice([1, 1, 2, 4, 8, 16, 32, 64]))   # R > 32 uses the upper half of the 64-bit rank sets
    epr = int(rng.integers(1, 1024 // R + 1)) if rng.random() < 0.3 else int(rng.integers(1, min(64, 1024 // R) + 1))
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


def _case_many_tiles(seed):
    """The shapes of _case(seed) with 700..6000 tokens (3 to 24 layout tiles) and hidden <= 1024."""
    inp, expand = _case(seed)
    c = inp["cfg"]
    rng = np.random.default_rng(50000 + seed)
    T = int(rng.integers(700, 6000))
    K, E = c.num_topk, c.num_experts
    idx = rng.integers(0, E, size=(T, K)).astype(np.int64)
    if rng.random() < 0.5:
        idx[rng.random((T, K)) < 0.05] = -1
    gen = torch.Generator().manual_seed(seed)
    w = W.softmax_weights(torch.randn(T, K, generator=gen))
    H = min(c.hidden, 1024)
    x = W.normal_bf16((T, H), gen)
    cfg = W.Config("tiles%d" % seed, T, H, E, K, "uniform", c.expert_alignment, c.zero_padding, c.fp8,
                   num_ranks=c.num_ranks, rank=c.rank)
    return dict(cfg=cfg, topk_idx=torch.from_numpy(idx), topk_weights=w, x=x, bias=None), expand


@pytest.mark.parametrize("seed", range(10))
def test_random_case_many_tiles(seed):
    _run_case(*_case_many_tiles(seed), seed)


@pytest.mark.parametrize("seed", range(NCASES))
def test_random_case(seed):
    _run_case(*_case(seed), seed)


def _run_case(inp, expand, seed):
    import combine_get_dispatch_03_amd as ep

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


def _rows_case(seed):
    rng = np.random.default_rng(5000 + seed)
    El = int(rng.integers(1, 129))
    N = int(rng.choice([0, 1, int(rng.integers(2, 256)), int(rng.integers(256, 900))]))
    K = int(rng.integers(1, 9))
    A = int(rng.choice([1, 4, 16, 128]))
    rb = 16 * int(rng.integers(1, 513))
    G = int(rng.choice([0, 0, int(rng.integers(1, 65))]))
    idx = rng.integers(0, El, size=(N, K)).astype(np.int64)
    if N:
        idx[rng.random((N, K)) < 0.4] = -1                            # entries owned by other ranks
        idx[rng.random(N) < 0.3] = -1                                 # rows not received
    rows = rng.integers(0, 256, size=(N, rb), dtype=np.uint8)
    sc = rng.random((N, G), dtype=np.float32) if G else None
    w = rng.random((N, K), dtype=np.float32)
    zp = bool(rng.random() < 0.5)
    return idx, El, A, rows, sc, w, zp


@pytest.mark.parametrize("seed", range(20))
def test_random_receiver_placement(seed):
    import combine_get_dispatch_03_amd as ep

    idx, El, A, rows, sc, w, zp = _rows_case(seed)
    N, rb = rows.shape
    print("[random rows %d] N=%d K=%d El=%d A=%d row_bytes=%d G=%d zp=%d" % (
        seed, N, idx.shape[1], El, A, rb, 0 if sc is None else sc.shape[1], zp), flush=True)
    h, _ = ep.ep_get_layout(torch.from_numpy(idx).to(DEV), El, 1, 0, A)
    cap = h.recv_capacity
    G = 0 if sc is None else sc.shape[1]
    out = Hn.fill_canaries(dict(
        recv_x=torch.empty((cap, rb), dtype=torch.uint8, device=DEV),
        recv_x_scales=torch.empty((cap, G), dtype=torch.float32, device=DEV) if G else None,
        recv_src_idx=torch.empty(cap, dtype=torch.int32, device=DEV),
        recv_topk_weights=torch.empty(cap, dtype=torch.float32, device=DEV)))
    ep.ep_dispatch_rows(h, torch.from_numpy(rows).to(DEV), torch.from_numpy(sc).to(DEV) if G else None,
                        torch.from_numpy(w).to(DEV), do_zero_padding=zp, out=out)
    lay = O.layout(idx, El, 1, 0, A)
    ref = O.dispatch_rows(rows, sc, idx, w, lay, El, A, zero_pad=zp, recv_fill=(Hn.CANARY_BYTE, Hn.CANARY_SCALE))
    got = Hn.to_np(out["recv_x"])
    assert np.array_equal(got, ref["recv_x"]), Hn._first_diff(got, ref["recv_x"])
    if G:
        assert np.array_equal(Hn.to_np(out["recv_x_scales"]).view(np.uint32), ref["recv_scales"].view(np.uint32))
    assert np.array_equal(Hn.to_np(out["recv_src_idx"]), ref["recv_src"])
    assert np.array_equal(Hn.to_np(out["recv_topk_weights"]).view(np.uint32), ref["recv_w"].view(np.uint32))


@pytest.mark.parametrize("seed", range(20))
def test_random_source_reduce(seed):
    import combine_get_dispatch_03_amd as ep

    rng = np.random.default_rng(7000 + seed)
    R = int(rng.choice([1, 2, 3, 4, 8, 16]))
    E = R * int(rng.integers(1, 33))
    T = int(rng.choice([0, 1, int(rng.integers(2, 300)), int(rng.integers(300, 1200))]))
    K = int(rng.integers(1, min(E, 8) + 1))
    H = 8 * int(rng.integers(1, 257))
    rank = int(rng.integers(0, R))
    with_local, with_bias = bool(rng.random() < 0.7), bool(rng.random() < 0.5)
    print("[random reduce %d] R=%d E=%d T=%d K=%d H=%d rank=%d local=%d bias=%d" % (
        seed, R, E, T, K, H, rank, with_local, with_bias), flush=True)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int64) if T else \
        np.zeros((0, K), np.int64)
    gen = torch.Generator().manual_seed(seed)
    parts = W.normal_bf16((R, T, H), gen)
    local = W.normal_bf16((T, H), gen) if with_local else None
    bias = W.normal_bf16((T, H), gen, 0.1) if with_bias else None
    h, _ = ep.ep_get_layout(torch.from_numpy(idx).to(DEV), E, R, rank, 1)
    out = ep.ep_combine_reduce(h, parts.to(DEV), local.to(DEV) if with_local else None,
                               bias.to(DEV) if with_bias else None, hidden=H)
    torch.cuda.synchronize()
    lay = O.layout(idx, E, R, rank, 1)
    ref = O.combine_reduce(W.bf16_bits(parts), lay["send_slot"], rank, W.bf16_bits(local) if with_local else None,
                           W.bf16_bits(bias) if with_bias else None)
    ok, mabs, mrel, nbad = Hn.combine_check(Hn.to_np(out), ref)
    assert ok, (mabs, mrel, nbad)


@pytest.mark.parametrize("K,rank,T,H", [(32, 0, 300, 616), (32, 63, 300, 616), (12, 17, 300, 616),
                                          (32, 5, 8200, 520)])
def test_source_reduce_64_ranks(K, rank, T, H):
    """The largest rank count: every lane of a wave reads a window row, and a token spread over many ranks has
    more returned rows than one unrolled batch holds.  With 300 tokens (a latency-bound grid) they are gathered
    in batches of 8; with 8200 tokens the grid is large enough for the waves to stream them one at a time.  H
    is not a multiple of 512, so the last segment of each row has idle lanes."""
    import combine_get_dispatch_03_amd as ep

    R, E = 64, 128
    rng = np.random.default_rng(9100 + K + rank)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int64)
    gen = torch.Generator().manual_seed(K * 100 + rank)
    parts = W.normal_bf16((R, T, H), gen)
    local = W.normal_bf16((T, H), gen)
    bias = W.normal_bf16((T, H), gen, 0.1)
    print("[reduce 64 ranks] K=%d rank=%d T=%d H=%d" % (K, rank, T, H), flush=True)
    h, _ = ep.ep_get_layout(torch.from_numpy(idx).to(DEV), E, R, rank, 1)
    out = ep.ep_combine_reduce(h, parts.to(DEV), local.to(DEV), bias.to(DEV), hidden=H)
    torch.cuda.synchronize()
    lay = O.layout(idx, E, R, rank, 1)
    nrows = (lay["send_slot"] >= 0).sum(axis=1)
    assert nrows.max() >= 8          # the streamed path is taken
    ref = O.combine_reduce(W.bf16_bits(parts), lay["send_slot"], rank, W.bf16_bits(local), W.bf16_bits(bias))
    ok, mabs, mrel, nbad = Hn.combine_check(Hn.to_np(out), ref)
    assert ok, (mabs, mrel, nbad)
