"""GPU parity: the HIP library (through the C ABI's Python binding) against the CPU oracle on the same seeded
inputs.  Layout and dispatch must match bit for bit (including rows that must stay untouched, checked with
canaries); combine must satisfy |gpu - oracle| <= 1e-2 + 8e-3 * |oracle| element-wise, and its closed forms
exactly.  Workloads are the five configurations of workloads/ at full size."""
import numpy as np
import pytest
import torch

import harness as Hn
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def ep():
    import combine_get_dispatch_03_amd as ep
    return ep


_cache = {}


def _run(ep, name):
    """Oracle and GPU layout + dispatch for one workload, cached for the module."""
    if name not in _cache:
        print("[parity] %s: inputs + oracle" % name, flush=True)
        inp = W.make_inputs(name)
        olay, od = Hn.oracle_run(inp)
        print("[parity] %s: gpu layout + dispatch" % name, flush=True)
        h, glay, gout = Hn.gpu_layout_dispatch(ep, inp, DEV)
        torch.cuda.synchronize()
        _cache[name] = (inp, olay, od, h, glay, gout)
    return _cache[name]


def test_single_hip_runtime(ep):
    libs = ep.hip_runtimes_loaded()
    assert len(libs) == 1, libs
    with open("/proc/self/maps") as f:
        assert ep.LIB_PATH in f.read()


def test_fp8_format_probe(ep):
    """One token whose group max is 448 (so inv = 1): codes must be the OCP e4m3fn codes of the values."""
    import json, os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e4m3_codes.json")))["cases"]
    keep = [c for c in cases if abs(c["value"]) <= 448.0
            and torch.tensor([c["value"]]).to(torch.bfloat16).float().item() == c["value"]]
    vals = [c["value"] for c in keep]
    codes = [c["code"] for c in keep]
    x = torch.zeros(1, 128, dtype=torch.float32)
    x[0, 0] = 448.0
    x[0, 1:1 + len(vals)] = torch.tensor(vals)
    xb = x.to(torch.bfloat16)
    assert torch.equal(xb.float(), x)             # every probe value is a bf16 value
    idx = torch.zeros(1, 1, dtype=torch.int64, device=DEV)
    h, _ = ep.ep_get_layout(idx, 1)
    d = ep.ep_dispatch(h, xb.to(DEV), None, fp8=True)
    q = d["recv_x"][0].cpu().numpy()
    assert int(q[0]) == 0x7E
    assert q[1:1 + len(vals)].tolist() == codes
    assert d["recv_x_scales"][0, 0].item() == 1.0


@pytest.mark.parametrize("name", W.ORDER)
def test_layout_parity(ep, name):
    inp, olay, od, h, glay, gout = _run(ep, name)
    Hn.assert_layout_equal(glay, olay, inp["cfg"])


@pytest.mark.parametrize("name", W.ORDER)
def test_dispatch_parity(ep, name):
    inp, olay, od, h, glay, gout = _run(ep, name)
    Hn.assert_dispatch_equal(gout, od, inp["cfg"])


@pytest.mark.parametrize("name", W.ORDER)
def test_combine_parity_random_y(ep, name):
    inp, olay, od, h, glay, gout = _run(ep, name)
    c = inp["cfg"]
    y = W.random_expert_outputs(h.recv_capacity, c.hidden, seed=100 + W.ORDER.index(name), device=DEV)
    bias = inp["bias"].to(DEV) if inp["bias"] is not None else None
    w = inp["topk_weights"].to(DEV)
    out, guard = Hn.guarded_tensor((c.num_tokens, c.hidden), torch.bfloat16, DEV)
    ep.ep_combine(h, y, w, bias, out=out)
    torch.cuda.synchronize()
    Hn.assert_guards(guard)
    ref = O.combine(Hn.to_np(y), olay["slot"], inp["topk_weights"].numpy(),
                    W.bf16_bits(inp["bias"]) if inp["bias"] is not None else None)
    ok, mabs, mrel, nbad = Hn.combine_check(Hn.to_np(out), ref)
    print("[combine %s] max_abs %.3g max_rel %.3g bad %d" % (name, mabs, mrel, nbad))
    assert ok, (mabs, mrel, nbad)


@pytest.mark.parametrize("name", ["tiny", "prefill", "ep8"])
def test_combine_closed_form_doubling(ep, name):
    """y = bf16(2 x[row_src]) and weights summing to 1: out == bf16(2 x) exactly for tokens with local slots
    whose local weights sum to 1 (all tokens when num_ranks == 1)."""
    inp, olay, od, h, glay, gout = _run(ep, name)
    c = inp["cfg"]
    y = Hn.closed_form_y(inp["x"], olay["row_src"], h.recv_capacity).to(DEV)
    out = ep.ep_combine(h, y, inp["topk_weights"].to(DEV))
    got = Hn.to_np(out)
    two_x = Hn.to_np((inp["x"].float() * 2).to(torch.bfloat16))
    if c.num_ranks == 1:
        assert np.array_equal(got, two_x)
    else:
        ref = O.combine(Hn.to_np(y), olay["slot"], inp["topk_weights"].numpy())
        ok, mabs, mrel, nbad = Hn.combine_check(got, ref)
        assert ok, (mabs, mrel, nbad)
        none_local = (olay["slot"] < 0).all(axis=1)
        assert (got[none_local] == 0).all()


def test_combine_unweighted_closed_form(ep):
    """Weights NULL (already-weighted rows): y = 2 x[row_src] with K = 8 gives exactly 16 x."""
    inp, olay, od, h, glay, gout = _run(ep, "prefill")
    y = Hn.closed_form_y(inp["x"], olay["row_src"], h.recv_capacity).to(DEV)
    out = ep.ep_combine(h, y, None)
    ref = (inp["x"].float() * 16).to(torch.bfloat16)
    assert np.array_equal(Hn.to_np(out), Hn.to_np(ref))


def test_round_trip_identity_bf16(ep):
    """BF16 dispatch, y = the dispatched rows, weights summing to 1: combine returns x bit for bit."""
    inp, olay, od, h, glay, gout = _run(ep, "tiny")
    out = ep.ep_combine(h, gout["recv_x"], inp["topk_weights"].to(DEV))
    assert np.array_equal(Hn.to_np(out), W.bf16_bits(inp["x"]))


def test_determinism(ep):
    inp = W.make_inputs("prefill")
    res = []
    for _ in range(2):
        h, glay, gout = Hn.gpu_layout_dispatch(ep, inp, DEV)
        y = W.random_expert_outputs(h.recv_capacity, 7168, seed=5, device=DEV)
        out = ep.ep_combine(h, y, inp["topk_weights"].to(DEV))
        torch.cuda.synchronize()
        res.append([Hn.to_np(t) for t in (glay["psum_num_recv_tokens_per_expert"], gout["recv_x"],
                                           gout["recv_x_scales"], gout["recv_src_idx"], out)])
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_cached_handle_new_x(ep):
    """The handle is reused for a second dispatch with new activations (cached use)."""
    inp = W.make_inputs("decode")
    c = inp["cfg"]
    h, glay, gout = Hn.gpu_layout_dispatch(ep, inp, DEV)
    x2 = W.normal_bf16((c.num_tokens, c.hidden), torch.Generator().manual_seed(77))
    out2 = Hn.dispatch_outputs_with_canary(ep, h, c.hidden, c.fp8, DEV)
    ep.ep_dispatch(h, x2.to(DEV), inp["topk_weights"].to(DEV), fp8=True, do_zero_padding=False, out=out2)
    inp2 = dict(inp, x=x2)
    olay, od = Hn.oracle_run(inp2)
    Hn.assert_dispatch_equal(out2, od, c)


def test_quantizer_sweep_all_bf16(ep):
    """Every finite bf16 value x, under group maxima spanning tiny (< 1e-4), subnormal-producing, ordinary and
    huge magnitudes: the FP8 codes and scales match the oracle bit for bit."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(O.bf16_to_f32(allb))
    xs = allb[fin]
    amaxes = np.array([2.0 ** -133, 1e-6, 5e-5, 1e-4, 1.5e-4, 0.01, 0.37, 1.0, 2.0, 3.1415, 7.5, 100.0, 448.0,
                       1e4, 3.3e38], np.float32)
    rows = []
    for am in amaxes:
        amb = W.bf16_bits(torch.tensor([am], dtype=torch.float32).to(torch.bfloat16))[0]
        amf = O.bf16_to_f32(np.array([amb], np.uint16))[0]
        sel = xs[np.abs(O.bf16_to_f32(xs)) <= amf]
        # groups of 128: slot 0 carries the group max, 127 values follow
        n = -(-len(sel) // 127)
        pad = np.zeros(n * 127, np.uint16)
        pad[: len(sel)] = sel
        g = np.concatenate([np.full((n, 1), amb, np.uint16), pad.reshape(n, 127)], axis=1)
        rows.append(g.reshape(-1))
    flat = np.concatenate(rows)
    H = 7168
    T = -(-flat.size // H)
    xb = np.zeros(T * H, np.uint16)
    xb[: flat.size] = flat
    xb = xb.reshape(T, H)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
    idx = torch.zeros(T, 1, dtype=torch.int64)
    h, _ = ep.ep_get_layout(idx.to(DEV), 1)
    d = ep.ep_dispatch(h, x.to(DEV), None, fp8=True)
    gq, gs = Hn.to_np(d["recv_x"])[:T], Hn.to_np(d["recv_x_scales"])[:T]
    for t in range(T):
        q, s = O.quantize_row(xb[t])
        assert np.array_equal(gq[t], q), (t, Hn._first_diff(gq[t], q))
        assert np.array_equal(gs[t].view(np.uint32), s.view(np.uint32)), t


def _quantize_on_gpu(ep, xb):
    """FP8 dispatch of bf16 bits xb [T, H] with every token routed to one expert: row t of the output is token t."""
    T = xb.shape[0]
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
    idx = torch.zeros(T, 1, dtype=torch.int64)
    h, _ = ep.ep_get_layout(idx.to(DEV), 1)
    out = Hn.dispatch_outputs_with_canary(ep, h, xb.shape[1], True, DEV)
    ep.ep_dispatch(h, x.to(DEV), None, fp8=True, out=out)
    torch.cuda.synchronize()
    Hn.assert_guards(out)
    return Hn.to_np(out["recv_x"])[:T], Hn.to_np(out["recv_x_scales"])[:T]


def test_quantizer_every_group_max(ep):
    """Every finite positive bf16 value (0x0001..0x7F7F, 32,639 of them) as a 128-channel group maximum, each
    heading 8 groups whose other 127 values are drawn from the bf16 codes between 0 and the maximum (magnitudes
    log-uniform, random signs; the first group of each maximum also holds -max, +0 and -0): codes and scales
    bit-equal to the oracle.  With the sweep above (every x under 15 maxima) this pins scale = amax / 448 and
    inv = 448 / amax for every maximum and the cast of x * inv across each maximum's range (33.4 M values)."""
    G_PER = 8
    maxima = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    n = maxima.size * G_PER
    m = np.repeat(maxima, G_PER)
    rng = np.random.default_rng(20240607)
    codes = np.minimum((rng.random((n, 127)) * (m[:, None].astype(np.float64) + 1)).astype(np.uint32), m[:, None])
    signs = (rng.random((n, 127)) < 0.5).astype(np.uint32) << 15
    groups = np.empty((n, 128), np.uint16)
    groups[:, 0] = m
    groups[:, 1:] = (codes | signs).astype(np.uint16)
    groups[::G_PER, 1] = maxima | 0x8000
    groups[::G_PER, 2] = 0x0000
    groups[::G_PER, 3] = 0x8000
    assert (np.abs(O.bf16_to_f32(groups)) <= O.bf16_to_f32(m)[:, None]).all()
    H = 7168
    flat = groups.reshape(-1)
    T = -(-flat.size // H)
    xb = np.zeros(T * H, np.uint16)
    xb[: flat.size] = flat
    xb = xb.reshape(T, H)
    print("[quantizer] %d groups, %d tokens" % (n, T), flush=True)
    gq, gs = _quantize_on_gpu(ep, xb)
    q, sc = O.quantize_row(xb.reshape(-1))
    q, sc = q.reshape(T, H), sc.reshape(T, H // 128)
    assert np.array_equal(gs.view(np.uint32), sc.view(np.uint32)), Hn._first_diff(gs.view(np.uint32),
                                                                                   sc.view(np.uint32))
    assert np.array_equal(gq, q), Hn._first_diff(gq, q)


def test_nonfinite_groups_do_not_disturb_others(ep):
    """Non-finite x (NaN, +-inf) has no defined e4m3 code here: the codes and the scale of the 128-channel group
    holding it are unspecified.  Every other group of the same token, every other token and everything past the
    outputs stay as they would be (bit-equal to the oracle; guard tails intact)."""
    T, H = 64, 7168
    xb = W.bf16_bits(W.normal_bf16((T, H), torch.Generator().manual_seed(9))).copy()
    planted = {(3, 5, 7): 0x7FC0,      # quiet NaN
               (3, 6, 0): 0xFFC0,      # negative quiet NaN, next group
               (10, 0, 0): 0x7F80,     # +inf, first group
               (20, 55, 127): 0xFF80,  # -inf, last group, last channel
               (40, 12, 64): 0x7F81,   # signalling NaN
               (41, 30, 1): 0x7F80}
    for (t, g, c), v in planted.items():
        xb[t, 128 * g + c] = v
    gq, gs = _quantize_on_gpu(ep, xb)
    q, sc = O.quantize_row(xb.reshape(-1))
    q, sc = q.reshape(T, H // 128, 128), sc.reshape(T, H // 128)
    gq = gq.reshape(T, H // 128, 128)
    keep = np.ones((T, H // 128), bool)
    for (t, g, _c) in planted:
        keep[t, g] = False
    assert np.array_equal(gq[keep], q[keep])
    assert np.array_equal(gs[keep].view(np.uint32), sc[keep].view(np.uint32))


# ---- edge cases -----------------------------------------------------------------------------------------

EDGE = [
    # T, K, E, R, rank, A, H, fp8, zero_pad, kind
    (0, 4, 8, 1, 0, 16, 256, False, True, "uniform"),
    (1, 1, 1, 1, 0, 1, 128, True, True, "uniform"),
    (1, 8, 256, 1, 0, 128, 7168, True, True, "uniform"),
    (300, 6, 64, 1, 0, 16, 384, True, True, "uniform"),        # ragged tile, H not a multiple of 1024
    (1000, 3, 24, 3, 2, 7, 136, False, True, "dup"),          # ragged, duplicates, H % 128 != 0 (BF16)
    (513, 32, 1024, 1, 0, 1, 8, False, False, "uniform"),     # K and E at their limits, tiny rows
    (257, 4, 128, 64, 63, 5, 256, True, False, "uniform"),    # 64 ranks, last rank
    (200, 5, 40, 4, 1, 1000, 1024, True, True, "invalid"),    # large alignment, -1 and invalid entries
    (4096, 8, 256, 8, 3, 128, 2048, True, True, "skew"),      # one hot expert owned by this rank
    (256, 8, 256, 4, 1, 64, 512, True, True, "uniform"),      # exactly one tile, with send windows
    (257, 3, 16, 2, 0, 8, 256, False, True, "invalid"),       # one token past a tile, BF16 windows
    (40, 4, 16, 1, 0, 8, 32768, False, True, "uniform"),      # largest hidden: 64 KiB BF16 rows
    (40, 4, 16, 2, 1, 8, 32768, True, True, "uniform"),       # largest hidden: 32 FP8 segments, windows
    (65536, 8, 256, 1, 0, 128, 128, True, True, "uniform"),   # 256 layout tiles
    (5, 1, 1, 1, 0, 65536, 8, False, True, "uniform"),        # largest alignment: 65,531 zero-padded rows
    (300, 2, 2, 2, 1, 65536, 128, True, True, "uniform"),     # largest alignment, FP8, two ranks
    (256, 32, 1024, 64, 5, 128, 256, True, True, "dup"),      # one full tile at the largest K, E and ranks
    (256, 32, 1024, 1, 0, 7, 128, False, True, "invalid"),    # one full tile, 1024 local experts, invalid ids
]


def _edge_inputs(T, K, E, kind, H, seed):
    gen = torch.Generator().manual_seed(seed)
    if kind == "dup":
        idx = torch.randint(0, E, (T, K), generator=gen)
    elif kind == "skew":
        idx = W.route_uniform_distinct(T, E, K, gen)
        idx[:, 0] = 3 * (E // 8) + 1                      # every token hits one expert of rank 3
        idx[:, 1:] = torch.where(idx[:, 1:] == 3 * (E // 8) + 1, 0, idx[:, 1:])
    else:
        idx = W.route_uniform_distinct(T, E, K, gen) if T > 0 else torch.zeros(0, K, dtype=torch.int64)
    if kind == "invalid" and T > 0:
        idx[::7, 0] = -1
        idx[3::11, K - 1] = E + 5
        idx[5::13, 1] = -9
    w = W.softmax_weights(torch.randn(T, K, generator=gen))
    x = W.normal_bf16((T, H), gen)
    return idx.contiguous(), w, x


@pytest.mark.parametrize("case", EDGE, ids=[str(i) for i in range(len(EDGE))])
def test_edge_cases(ep, case):
    T, K, E, R, rank, A, H, fp8, zp, kind = case
    print("[edge] T=%d K=%d E=%d R=%d rank=%d A=%d H=%d fp8=%d zp=%d %s" % case, flush=True)
    idx, w, x = _edge_inputs(T, K, E, kind, H, seed=T + K + E)
    cfg = W.Config("edge", T, H, E, K, kind, A, zp, fp8, num_ranks=R, rank=rank)
    inp = dict(cfg=cfg, topk_idx=idx, topk_weights=w, x=x, bias=None)
    olay, od = Hn.oracle_run(inp)
    h, glay, gout = Hn.gpu_layout_dispatch(ep, inp, DEV)
    Hn.assert_layout_equal(glay, olay, cfg)
    Hn.assert_dispatch_equal(gout, od, cfg)
    y = W.random_expert_outputs(h.recv_capacity, H, seed=T, device=DEV)
    bias = W.normal_bf16((T, H), torch.Generator().manual_seed(1), 0.1)
    out, guard = Hn.guarded_tensor((T, H), torch.bfloat16, DEV)
    ep.ep_combine(h, y, w.to(DEV), bias.to(DEV), out=out)
    torch.cuda.synchronize()
    Hn.assert_guards(guard)
    ref = O.combine(Hn.to_np(y), olay["slot"], w.numpy(), W.bf16_bits(bias))
    ok, mabs, mrel, nbad = Hn.combine_check(Hn.to_np(out), ref)
    assert ok, (mabs, mrel, nbad)


def test_validation_errors(ep):
    inp = W.make_inputs("decode")
    h, glay, gout = Hn.gpu_layout_dispatch(ep, inp, DEV)
    x = inp["x"].to(DEV)
    short = ep.alloc_dispatch_outputs(h, 7168, True, device=DEV, recv_capacity=h.recv_capacity - 1)
    with pytest.raises(ep.EPError, match="recv_capacity"):
        ep.ep_dispatch(h, x, None, fp8=True, out=short)
    short_tm = ep.alloc_dispatch_outputs(h, 7168, True, device=DEV, recv_capacity=h.num_tokens - 1,
                                         do_expand=False)
    with pytest.raises(ep.EPError, match="recv_capacity"):
        ep.ep_dispatch(h, x, None, fp8=True, do_expand=False, out=short_tm)
    with pytest.raises(ep.EPError, match="y_rows"):
        ep.ep_combine_tokens(h, torch.zeros(h.num_tokens - 1, 7168, dtype=torch.bfloat16, device=DEV))
    y = torch.zeros(h.recv_capacity - 1, 7168, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ep.EPError, match="y_rows"):
        ep.ep_combine(h, y, None)
    with pytest.raises(ep.EPError, match="hidden"):
        ep.ep_dispatch(h, torch.zeros(128, 100, dtype=torch.bfloat16, device=DEV), None, fp8=True)
