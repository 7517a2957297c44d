"""Pins for the oracle's receiver-side placement and source-side reduce.

(1) Placement of pre-quantised rows equals the sender's own dispatch (two code paths: quantise-and-scatter vs
    place-received-rows) on the same layout.
(2) The expert-parallel decomposition identity: sending every token's row to the ranks holding its experts,
    placing it there, combining each rank's weighted outputs per token, returning those partial rows and
    adding them up gives the same result as combining all experts at once:
        out[t] = sum_k w[t,k] * f(x[t]) + bias[t]
    with the expert function f = bf16(dequantise(quantise(x))) (every expert the identity on its input).  The
    only difference is the BF16 rounding of the returned partial rows, bounded below.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def _quantised(x_bits):
    q = np.empty((x_bits.shape[0], x_bits.shape[1]), np.uint8)
    s = np.empty((x_bits.shape[0], x_bits.shape[1] // 128), np.float32)
    for t in range(x_bits.shape[0]):
        q[t], s[t] = O.quantize_row(x_bits[t])
    return q, s


def _dequant(q, s):
    return O.e4m3_decode(q).astype(np.float64) * np.repeat(s.astype(np.float64), 128, axis=1)


@pytest.mark.parametrize("fp8", [True, False])
def test_rows_placement_equals_dispatch(fp8):
    gen = torch.Generator().manual_seed(21)
    T, K, E, H, A = 70, 3, 12, 256, 8
    idx = W.route_uniform_distinct(T, E, K, gen).numpy()
    idx[5, 1] = -1
    w = W.softmax_weights(torch.randn(T, K, generator=gen)).numpy()
    x = W.bf16_bits(W.normal_bf16((T, H), gen))
    lay = O.layout(idx, E, 1, 0, A)
    d = O.dispatch(x, idx, w, lay, E, 1, 0, A, fp8=fp8, zero_pad=True, recv_fill=(0xA5, -3.0))
    if fp8:
        rows, sc = _quantised(x)
    else:
        rows, sc = x.view(np.uint8).reshape(T, 2 * H), None
    r = O.dispatch_rows(rows, sc, idx, w, lay, E, A, zero_pad=True, recv_fill=(0xA5, -3.0))
    assert np.array_equal(r["recv_x"], d["recv_x"].view(np.uint8).reshape(r["recv_x"].shape))
    if fp8:
        assert np.array_equal(r["recv_scales"], d["recv_scales"])
    valid = lay["row_src"] >= 0
    assert np.array_equal(r["recv_src"][valid], lay["row_src"][valid])        # received row index = token
    assert np.array_equal(r["recv_w"], d["recv_w"])


def ep_roundtrip_oracle(ranks_inputs, E, R, A, K, H, bias_list):
    """Run the whole expert-parallel round trip through the oracle.  ranks_inputs[s] = (idx, w, x_bits)."""
    T = ranks_inputs[0][0].shape[0]
    El = E // R
    lays, disp = [], []
    for s, (idx, w, x) in enumerate(ranks_inputs):
        lay = O.layout(idx, E, R, s, A)
        lays.append(lay)
        disp.append(O.dispatch(x, idx, w, lay, E, R, s, A, fp8=True, zero_pad=False))
    partial_windows = np.zeros((R, R, T, H), np.uint16)      # [source s][rank r] window
    local_out = []
    for r in range(R):
        # rows received by rank r: window r of every other source, rows beyond its count are absent (-1)
        rows = np.zeros((R * T, H), np.uint8)
        sc = np.zeros((R * T, H // 128), np.float32)
        tk = np.full((R * T, K), -1, np.int64)
        tw = np.zeros((R * T, K), np.float32)
        for s in range(R):
            if s == r:
                continue
            n = int(lays[s]["ntok_rank"][r])
            rows[s * T:s * T + n] = disp[s]["send_x"][r, :n]
            sc[s * T:s * T + n] = disp[s]["send_scales"][r, :n]
            tk[s * T:s * T + n] = disp[s]["send_topk_idx"][r, :n]
            tw[s * T:s * T + n] = disp[s]["send_topk_w"][r, :n]
        rl = O.layout(tk, El, 1, 0, A)
        rd = O.dispatch_rows(rows, sc, tk, tw, rl, El, A, zero_pad=False)
        # expert compute: every expert returns its input, dequantised, in BF16
        used = int(rl["psum"][-1])
        y = np.zeros((rl["cap"], H), np.uint16)
        ok = rd["recv_src"][:used] >= 0
        y[:used][ok] = O.f64_to_bf16(_dequant(rd["recv_x"][:used][ok], rd["recv_scales"][:used][ok]))
        part = O.f64_to_bf16(O.combine(y, rl["slot"], tw))         # one BF16 row per received row
        for s in range(R):
            partial_windows[s, r] = part[s * T:(s + 1) * T]
        # rank r's own tokens through its local expert-major rows
        own = disp[r]
        yl = np.zeros((lays[r]["cap"], H), np.uint16)
        used_l = int(lays[r]["psum"][-1])
        okl = own["recv_src"][:used_l] >= 0
        yl[:used_l][okl] = O.f64_to_bf16(_dequant(own["recv_x"][:used_l][okl], own["recv_scales"][:used_l][okl]))
        local_out.append(O.f64_to_bf16(O.combine(yl, lays[r]["slot"], ranks_inputs[r][1])))
    outs = []
    for s in range(R):
        outs.append(O.combine_reduce(partial_windows[s], lays[s]["send_slot"], s, local_out[s], bias_list[s]))
    return outs


def test_ep_roundtrip_identity():
    gen = torch.Generator().manual_seed(33)
    R, T, E, K, H, A = 4, 40, 16, 3, 256, 4
    ins, biases = [], []
    for s in range(R):
        idx = W.route_uniform_distinct(T, E, K, gen).numpy()
        w = W.softmax_weights(torch.randn(T, K, generator=gen)).numpy()
        x = W.bf16_bits(W.normal_bf16((T, H), gen))
        ins.append((idx, w, x))
        biases.append(W.bf16_bits(W.normal_bf16((T, H), gen, 0.1)))
    outs = ep_roundtrip_oracle(ins, E, R, A, K, H, biases)
    for s in range(R):
        idx, w, x = ins[s]
        q, sc = _quantised(x)
        g = O.bf16_to_f32(O.f64_to_bf16(_dequant(q, sc))).astype(np.float64)   # every expert's BF16 output
        ref = w.astype(np.float64).sum(axis=1, keepdims=True) * g + O.bf16_to_f32(biases[s]).astype(np.float64)
        # each returned partial (and the local part) w_r * g was rounded to BF16 once, |err| <= 2^-8 |w_r g|,
        # and the weights sum to 1: |err| <= 2^-8 |g| (+ float32 slack of the weight sum)
        bound = 2.0 ** -8 * np.abs(g) * (1 + 1e-6) + 1e-30
        assert (np.abs(outs[s] - ref) <= bound).all()
