"""Pins for the oracle's dispatch (quantiser, placement, padding, send windows) and combine.

The quantiser is pinned by a hand-worked group (tests/golden/quantizer_group.json), by its dequantisation
bound and by the group maximum mapping to +-448.  Placement is checked as a gather (row r holds token
row_src[r]), the opposite formulation of the oracle's scatter.  Combine is checked against a dense
scatter-matrix product (numpy matmul) and against the closed forms of the pages' round trip.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_quantizer_golden_group():
    g = json.load(open(os.path.join(GOLD, "quantizer_group.json")))
    x = np.full(128, g["other_entries_bf16_bits"], np.uint16)
    for e in g["entries"]:
        x[e["index"]] = e["x_bf16_bits"]
    q, s = O.quantize_row(x)
    assert s[0] == np.float32(g["amax"]) / np.float32(448.0)
    for e in g["entries"]:
        assert int(q[e["index"]]) == e["code"], e
    others = np.setdiff1d(np.arange(128), [e["index"] for e in g["entries"]])
    assert (q[others] == 0).all()


def test_quantizer_bound_and_amax_code():
    gen = torch.Generator().manual_seed(1)
    x = W.normal_bf16((64, 1024), gen)
    x[3, :128] = 0                       # an all-zero group: scale from the 1e-4 floor, all codes zero
    x[5, 128:256] *= 1e-6                # a group below the floor
    bits = W.bf16_bits(x)
    xf = O.bf16_to_f32(bits).astype(np.float64)
    for r in range(bits.shape[0]):
        q, s = O.quantize_row(bits[r])
        deq = O.e4m3_decode(q).astype(np.float64)
        for gi in range(8):
            sl = slice(128 * gi, 128 * gi + 128)
            xs = xf[r, sl]
            amax = np.abs(xs).max()
            sc = float(s[gi])
            assert sc == np.float32(max(np.float32(amax), np.float32(1e-4))) / np.float32(448)
            err = np.abs(deq[sl] * sc - xs)
            bound = np.maximum(2.0 ** -4 * np.abs(xs), 2.0 ** -10 * sc) + 2.0 ** -20 * np.abs(xs)
            assert (err <= bound).all()
            if amax >= 1e-4:
                j = int(np.argmax(np.abs(xs)))
                assert abs(float(deq[sl][j])) == 448.0
            if amax == 0:
                assert (q[sl] == 0).all()


def _layout_dispatch(name=None, T=None, K=None, E=None, R=1, rank=0, A=1, H=256, fp8=False, zero_pad=True,
                     seed=0):
    if name is not None:
        inp = W.make_inputs(name)
        c = inp["cfg"]
        idx, w, x = inp["topk_idx"].numpy(), inp["topk_weights"].numpy(), W.bf16_bits(inp["x"])
        E, R, rank, A, fp8, zero_pad = c.num_experts, c.num_ranks, c.rank, c.expert_alignment, c.fp8, c.zero_padding
    else:
        gen = torch.Generator().manual_seed(seed)
        idx = W.route_uniform_distinct(T, E, K, gen).numpy()
        w = W.softmax_weights(torch.randn(T, K, generator=gen)).numpy()
        x = W.bf16_bits(W.normal_bf16((T, H), gen))
    lay = O.layout(idx, E, R, rank, A)
    d = O.dispatch(x, idx, w, lay, E, R, rank, A, fp8=fp8, zero_pad=zero_pad, recv_fill=(0xA5, -3.0))
    return idx, w, x, lay, d, dict(E=E, R=R, rank=rank, A=A, fp8=fp8, zero_pad=zero_pad)


@pytest.mark.parametrize("zero_pad", [True, False])
def test_bf16_dispatch_is_a_gather_of_row_src(zero_pad):
    idx, w, x, lay, d, p = _layout_dispatch(T=50, K=3, E=6, A=8, H=64, zero_pad=zero_pad, seed=2)
    used = lay["psum"][-1]
    rs = lay["row_src"]
    for r in range(lay["cap"]):
        if r < used and rs[r] >= 0:
            assert np.array_equal(d["recv_x"][r], x[rs[r]])
            assert d["recv_src"][r] == rs[r]
            k = int(np.nonzero(lay["slot"][rs[r]] == r)[0][0])
            assert d["recv_w"][r] == w[rs[r], k]
        elif r < used:                           # padding row
            fill = 0 if zero_pad else 0xA5A5
            assert (d["recv_x"][r] == fill).all()
            assert d["recv_src"][r] == -1 and d["recv_w"][r] == 0.0
        else:                                    # past the used rows: untouched
            assert (d["recv_x"][r] == 0xA5A5).all()
            assert d["recv_src"][r] == -7 and d["recv_w"][r] == -7.0


def test_fp8_dispatch_rows_and_pads():
    idx, w, x, lay, d, p = _layout_dispatch(T=40, K=4, E=8, A=16, H=384, fp8=True, zero_pad=True, seed=3)
    used = lay["psum"][-1]
    xf = O.bf16_to_f32(x).astype(np.float64)
    for r in range(used):
        t = lay["row_src"][r]
        if t < 0:
            assert (d["recv_x"][r] == 0).all() and (d["recv_scales"][r] == 0).all()
            continue
        deq = O.e4m3_decode(d["recv_x"][r]).astype(np.float64) * np.repeat(d["recv_scales"][r], 128)
        assert (np.abs(deq - xf[t]) <= np.maximum(2.0 ** -4 * np.abs(xf[t]), 2.0 ** -10 * np.repeat(
            d["recv_scales"][r], 128)) + 2.0 ** -20 * np.abs(xf[t])).all()
    # every copy of one token is the same bytes
    for t in range(idx.shape[0]):
        rows = [s for s in lay["slot"][t] if s >= 0]
        for s in rows[1:]:
            assert np.array_equal(d["recv_x"][s], d["recv_x"][rows[0]])
    assert (d["recv_x"][used:] == 0xA5).all()


def test_send_windows():
    idx, w, x, lay, d, p = _layout_dispatch(T=64, K=4, E=16, R=4, rank=1, A=4, H=256, fp8=True, zero_pad=False,
                                            seed=4)
    T, K = idx.shape
    epr = 4
    for r in range(4):
        toks = np.nonzero(lay["in_rank"][:, r])[0]
        if r == 1:
            assert (d["send_x"][r] == 0xA5).all()
            continue
        for j, t in enumerate(toks):
            q, s = O.quantize_row(x[t])
            assert np.array_equal(d["send_x"][r, j], q) and np.array_equal(d["send_scales"][r, j], s)
            assert d["send_src"][r, j] == t
            exp_idx = [int(e) - r * epr if r * epr <= e < (r + 1) * epr else -1 for e in idx[t]]
            assert d["send_topk_idx"][r, j].tolist() == exp_idx
            assert np.array_equal(d["send_topk_w"][r, j], w[t])
        assert (d["send_x"][r, len(toks):] == 0xA5).all()
        assert (d["send_src"][r, len(toks):] == -7).all()


def _dense_combine(y_bits, slot, w, bias_bits, rows):
    T, K = slot.shape
    S = np.zeros((T, rows))
    for t in range(T):
        for k in range(K):
            if slot[t, k] >= 0:
                S[t, slot[t, k]] += 1.0 if w is None else float(w[t, k])
    out = S @ O.bf16_to_f32(y_bits[:rows]).astype(np.float64)
    if bias_bits is not None:
        out += O.bf16_to_f32(bias_bits).astype(np.float64)
    return out


@pytest.mark.parametrize("weighted,with_bias", [(True, False), (False, False), (True, True)])
def test_combine_vs_dense_matmul(weighted, with_bias):
    gen = torch.Generator().manual_seed(9)
    T, K, E, H, A = 33, 3, 5, 40, 4
    idx = W.route_uniform_distinct(T, E, K, gen).numpy()
    idx[4, 1] = -1
    w = W.softmax_weights(torch.randn(T, K, generator=gen)).numpy()
    lay = O.layout(idx, E, 1, 0, A)
    y = W.bf16_bits(W.normal_bf16((lay["cap"], H), gen))
    bias = W.bf16_bits(W.normal_bf16((T, H), gen, 0.1)) if with_bias else None
    got = O.combine(y, lay["slot"], w if weighted else None, bias)
    ref = _dense_combine(y, lay["slot"], w if weighted else None, bias, lay["cap"])
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_round_trip_identity():
    """y = dispatched BF16 rows and weights summing to 1: the combine returns x (after BF16 rounding)."""
    idx, w, x, lay, d, p = _layout_dispatch("tiny")
    out = O.combine(d["recv_x"], lay["slot"], w, None)
    assert np.array_equal(O.f64_to_bf16(out), x)


def test_closed_forms_tiny():
    idx, w, x, lay, d, p = _layout_dispatch("tiny")
    y = np.zeros_like(d["recv_x"])
    rows = lay["row_src"] >= 0
    y[rows] = O.f64_to_bf16(2.0 * O.bf16_to_f32(x[lay["row_src"][rows]]).astype(np.float64))
    out = O.combine(y, lay["slot"], w, None)
    assert np.array_equal(O.f64_to_bf16(out), O.f64_to_bf16(2.0 * O.bf16_to_f32(x)))
    out_u = O.combine(d["recv_x"], lay["slot"], None, None)       # unweighted: K copies of x
    assert np.array_equal(out_u, idx.shape[1] * O.bf16_to_f32(x).astype(np.float64))


def test_token_without_local_expert_gets_bias():
    idx = np.array([[0, 1], [2, 3]], np.int64)
    lay = O.layout(idx, num_experts=4, num_ranks=2, rank=0, expert_alignment=1)
    H = 8
    y = np.full((lay["cap"], H), 0x3F80, np.uint16)              # 1.0
    bias = np.full((2, H), 0x4000, np.uint16)                    # 2.0
    out = O.combine(y, lay["slot"], np.array([[0.25, 0.75], [0.5, 0.5]], np.float32), bias)
    assert (out[0] == 3.0).all() and (out[1] == 2.0).all()


@pytest.mark.parametrize("fp8,R,rank", [(False, 1, 0), (True, 4, 2), (False, 3, 0)])
def test_token_major_dispatch(fp8, R, rank):
    """do_expand off: one row per token with a local expert, ascending token order (a gather over the tokens
    in this rank, brute force), local expert ids or -1 per entry, the token's weights; send windows are
    the same bytes as under the expert-major dispatch."""
    gen = torch.Generator().manual_seed(40 + R)
    T, K, E, H, A = 57, 3, 12, 256, 4
    idx = W.route_uniform_distinct(T, E, K, gen).numpy()
    idx[7, :] = -1                                   # a token with no expert at all
    w = W.softmax_weights(torch.randn(T, K, generator=gen)).numpy()
    x = W.bf16_bits(W.normal_bf16((T, H), gen))
    lay = O.layout(idx, E, R, rank, A)
    d = O.dispatch(x, idx, w, lay, E, R, rank, A, fp8=fp8, recv_fill=(0xA5, -3.0), do_expand=False)
    e = O.dispatch(x, idx, w, lay, E, R, rank, A, fp8=fp8, recv_fill=(0xA5, -3.0), do_expand=True)
    epr, lo = E // R, rank * (E // R)
    toks = [t for t in range(T) if any(lo <= v < lo + epr for v in idx[t])]
    assert len(toks) == int(lay["ntok_rank"][rank])
    for j, t in enumerate(toks):
        if fp8:
            q, s = O.quantize_row(x[t])
            assert np.array_equal(d["recv_x"][j], q) and np.array_equal(d["recv_scales"][j], s)
        else:
            assert np.array_equal(d["recv_x"][j], x[t])
        assert d["recv_src"][j] == t
        assert d["recv_topk_idx"][j].tolist() == [int(v) - lo if lo <= v < lo + epr else -1 for v in idx[t]]
        assert np.array_equal(d["recv_w"][j], w[t])
        # the same bytes as every expert-major copy of the token
        for s_ in lay["slot"][t]:
            if s_ >= 0:
                assert np.array_equal(e["recv_x"][s_], d["recv_x"][j])
    n = len(toks)
    assert (d["recv_x"][n:].view(np.uint8) == 0xA5).all()
    assert (d["recv_src"][n:] == -7).all() and (d["recv_topk_idx"][n:] == -7).all()
    if R > 1:
        for k in ("send_x", "send_scales", "send_src", "send_topk_idx", "send_topk_w"):
            if e[k] is not None:
                assert np.array_equal(d[k], e[k]), k
        assert (d["send_x"][rank].view(np.uint8) == 0xA5).all()      # no window towards this rank


def test_combine_tokens_closed_form():
    """Token-major combine: row j of y holds the value j + 1 (exact in BF16 for j < 256), so each token's
    output names the row it gathered; tokens without a local expert get exactly the bias."""
    idx = np.array([[0, 5], [4, 5], [1, 2], [6, 7], [3, 4]], np.int64)
    R, rank = 2, 0
    lay = O.layout(idx, num_experts=8, num_ranks=R, rank=rank, expert_alignment=1)
    H = 16
    y = O.f64_to_bf16(np.repeat(np.arange(1, 6, dtype=np.float64)[:, None], H, axis=1))
    bias = np.full((5, H), 0x3F00, np.uint16)        # 0.5
    out = O.combine_tokens(y, lay["send_slot"], rank, bias)
    # tokens 0, 2, 4 hold experts of rank 0 (0..3): rows 0, 1, 2; tokens 1 and 3 none
    assert out[:, 0].tolist() == [1.5, 0.5, 2.5, 0.5, 3.5]
    assert (out == out[:, :1]).all()
    out_nb = O.combine_tokens(y, lay["send_slot"], rank)
    assert out_nb[:, 0].tolist() == [1.0, 0.0, 2.0, 0.0, 3.0]
