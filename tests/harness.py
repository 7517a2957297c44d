"""Shared helpers of the parity tests: run one workload through the oracle and through the HIP library (via the
Python binding of the C ABI) on the same seeded inputs, and compare.

The oracle side gets only the seeded inputs (workloads/) and its own layout; no value from the HIP path ever
feeds it.  Expert outputs y are drawn by torch's seeded generator or built from x and the oracle's row map.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import workloads as W

CANARY_BYTE = 0xA5          # fill of receive / send buffers before dispatch, to catch stray or missing writes
CANARY_SCALE = -3.0
CANARY_I32 = -7
CANARY_F32 = -7.0
ATOL, RTOL = 1e-2, 8e-3     # combine tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle|


GUARD_ROWS = 2              # rows of canary past the end of every guarded output


class Guarded(dict):
    """Output tensors, each the leading part of a larger buffer whose tail (at least GUARD_ROWS rows past the
    documented size, and at least 256 elements) no call may touch: a store past the end of an output lands in
    the tail and is caught by assert_guards."""

    def __init__(self, *a, **kw):
        super().__init__(*a, **kw)
        self.parents = {}       # key -> (parent buffer, numel of the view)


def _guarded_empty(shape, dtype, device):
    shape = tuple(int(d) for d in shape)
    n = int(np.prod(shape)) if shape else 1
    row = shape[-1] if len(shape) > 1 else 1
    parent = torch.empty(n + max(GUARD_ROWS * row, 256), dtype=dtype, device=device)
    return parent[:n].view(shape), parent, n


def guard(o):
    """The same outputs (shapes and dtypes) as views into guarded buffers."""
    g = Guarded()
    for k, t in o.items():
        if t is None:
            g[k] = None
            continue
        v, parent, n = _guarded_empty(t.shape, t.dtype, t.device)
        g[k] = v
        g.parents[k] = (parent, n)
    return g


def guarded_tensor(shape, dtype, device, key="out"):
    """One guarded, canary-filled output tensor; returns (tensor, Guarded dict holding it)."""
    g = Guarded()
    v, parent, n = _guarded_empty(shape, dtype, device)
    g[key] = v
    g.parents[key] = (parent, n)
    fill_canaries(g)
    return v, g


def dispatch_outputs_with_canary(ep, h, hidden, fp8, dev, do_expand=True):
    """Dispatch output tensors, pre-filled with canaries (the binding itself never initialises them), each with a
    canary tail past its end."""
    return fill_canaries(guard(ep.alloc_dispatch_outputs(h, hidden, fp8, device=dev, do_expand=do_expand)))


def layout_outputs_with_canary(T, E, R, dev):
    El = E // R
    o = dict(num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=dev),
             num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=dev),
             is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=dev),
             psum_num_recv_tokens_per_expert=torch.empty(El + 1, dtype=torch.int32, device=dev),
             num_invalid_topk=torch.empty(1, dtype=torch.int32, device=dev))
    return fill_canaries(guard(o))


def _canary_fill(t, key):
    if t.dtype in (torch.uint8,):
        t.fill_(CANARY_BYTE)
    elif t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(np.int16(np.uint16(CANARY_BYTE * 257).view(np.int16)))
    elif t.dtype == torch.float32:
        t.fill_(CANARY_SCALE if "scales" in key else CANARY_F32)
    else:
        t.fill_(CANARY_I32)


def fill_canaries(o):
    for k, t in o.items():
        if t is None:
            continue
        if isinstance(o, Guarded) and k in o.parents:
            _canary_fill(o.parents[k][0], k)      # the tail too
        else:
            _canary_fill(t, k)
    return o


def assert_guards(o):
    """Every guarded output's tail still holds its canary."""
    if not isinstance(o, Guarded):
        return
    for k, (parent, n) in o.parents.items():
        tail = parent[n:]
        ref = torch.empty_like(tail)
        _canary_fill(ref, k)
        if tail.dtype == torch.bfloat16:
            tail, ref = tail.view(torch.int16), ref.view(torch.int16)
        elif tail.dtype == torch.float32:
            tail, ref = tail.view(torch.int32), ref.view(torch.int32)
        bad = (tail != ref).nonzero()
        assert bad.numel() == 0, "%s: %d element(s) written past its end, first at +%d" % (
            k, bad.shape[0], int(bad[0, 0]))


def to_np(t):
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def oracle_run(inp, recv_fill=True, do_expand=True):
    c = inp["cfg"]
    idx = inp["topk_idx"].numpy()
    w = inp["topk_weights"].numpy()
    x = W.bf16_bits(inp["x"])
    lay = O.layout(idx, c.num_experts, c.num_ranks, c.rank, c.expert_alignment)
    d = O.dispatch(x, idx, w, lay, c.num_experts, c.num_ranks, c.rank, c.expert_alignment, fp8=c.fp8,
                   zero_pad=c.zero_padding, recv_fill=(CANARY_BYTE, CANARY_SCALE) if recv_fill else None,
                   do_expand=do_expand)
    return lay, d


def gpu_layout_dispatch(ep, inp, dev="cuda", do_expand=True):
    c = inp["cfg"]
    idx = inp["topk_idx"].to(dev)
    lay_out = layout_outputs_with_canary(c.num_tokens, c.num_experts, c.num_ranks, dev)
    h, lay = ep.ep_get_layout(idx, c.num_experts, c.num_ranks, c.rank, c.expert_alignment, outputs=lay_out)
    out = dispatch_outputs_with_canary(ep, h, c.hidden, c.fp8, dev, do_expand=do_expand)
    ep.ep_dispatch(h, inp["x"].to(dev), inp["topk_weights"].to(dev), fp8=c.fp8, do_expand=do_expand,
                   do_zero_padding=c.zero_padding, out=out)
    return h, lay, out


def assert_layout_equal(glay, olay, c):
    assert_guards(glay)
    assert np.array_equal(to_np(glay["num_tokens_per_expert"]), olay["cnt"])
    assert np.array_equal(to_np(glay["num_tokens_per_rank"]), olay["ntok_rank"])
    assert np.array_equal(to_np(glay["is_token_in_rank"]), olay["in_rank"])
    assert np.array_equal(to_np(glay["psum_num_recv_tokens_per_expert"]), olay["psum"])
    assert int(to_np(glay["num_invalid_topk"])[0]) == int(olay["num_invalid"][0])


def assert_dispatch_equal(gout, od, c):
    """Bit-exact comparison of every dispatch output, including untouched (canary) rows and the guard tails."""
    assert_guards(gout)
    gx = to_np(gout["recv_x"])
    if c.fp8:
        assert np.array_equal(gx, od["recv_x"]), _first_diff(gx, od["recv_x"])
        gs = to_np(gout["recv_x_scales"])
        assert np.array_equal(gs.view(np.uint32), od["recv_scales"].view(np.uint32)), _first_diff(gs, od["recv_scales"])
    else:
        assert np.array_equal(gx, od["recv_x"]), _first_diff(gx, od["recv_x"])
    assert np.array_equal(to_np(gout["recv_src_idx"]), od["recv_src"])
    assert np.array_equal(to_np(gout["recv_topk_weights"]).view(np.uint32), od["recv_w"].view(np.uint32))
    if od.get("recv_topk_idx") is not None:
        assert np.array_equal(to_np(gout["recv_topk_idx"]), od["recv_topk_idx"])
    if od.get("send_x") is not None:
        sx = to_np(gout["send_x"])
        assert np.array_equal(sx.reshape(od["send_x"].shape).view(np.uint8), od["send_x"].view(np.uint8))
        if c.fp8:
            assert np.array_equal(to_np(gout["send_x_scales"]).view(np.uint32), od["send_scales"].view(np.uint32))
        assert np.array_equal(to_np(gout["send_src_idx"]), od["send_src"])
        assert np.array_equal(to_np(gout["send_topk_idx"]), od["send_topk_idx"])
        assert np.array_equal(to_np(gout["send_topk_weights"]).view(np.uint32), od["send_topk_w"].view(np.uint32))


def _first_diff(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        return "shape %s vs %s" % (a.shape, b.shape)
    d = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
    if d.size == 0:
        return "equal"
    i = d[0]
    return "%d mismatches; first at flat %d (row %d): gpu %r oracle %r" % (
        d.size, i, i // (a.shape[-1] if a.ndim > 1 else 1), a.reshape(-1)[i], b.reshape(-1)[i])


def combine_check(gout_bits, oref, atol=ATOL, rtol=RTOL):
    """Element-wise |g - o| <= atol + rtol*|o|; returns (ok, max_abs, max_rel, n_bad)."""
    g = O.bf16_to_f32(gout_bits).astype(np.float64)
    err = np.abs(g - oref)
    bad = err > atol + rtol * np.abs(oref)
    rel = err / np.maximum(np.abs(oref), 1e-30)
    return (not bad.any()), float(err.max(initial=0.0)), float(rel.max(initial=0.0)), int(bad.sum())


def closed_form_y(x, row_src, rows):
    """y[row] = bf16(2 * x[row_src[row]]) for valid rows, 0 elsewhere; x is a bf16 CPU tensor, doubling is
    exact in bf16."""
    y = torch.zeros((rows, x.shape[1]), dtype=torch.bfloat16)
    rs = torch.from_numpy(row_src[:rows].astype(np.int64))
    valid = rs >= 0
    y[valid] = (x[rs[valid]].float() * 2.0).to(torch.bfloat16)
    return y
