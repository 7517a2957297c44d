"""Property-based pins of the oracle (hypothesis): on arbitrary small routing tables, including -1, out-of-range
ids and duplicates, the oracle's layout equals brute-force recounts, its permutation equals numpy's stable argsort,
its per-rank token rows are dense in token order, and its dispatch + unweighted combine of a row-identity payload
returns K_local copies of each row (every routed entry is placed exactly once)."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O


@st.composite
def tables(draw):
    R = draw(st.sampled_from([1, 2, 3, 4, 8]))
    epr = draw(st.integers(1, 6))
    E = R * epr
    T = draw(st.integers(0, 40))
    K = draw(st.integers(1, 6))
    A = draw(st.sampled_from([1, 2, 3, 8, 16]))
    rank = draw(st.integers(0, R - 1))
    vals = st.one_of(st.integers(0, E - 1), st.integers(0, E - 1), st.just(-1), st.integers(-5, E + 5))
    idx = np.array(draw(st.lists(vals, min_size=T * K, max_size=T * K)), np.int64).reshape(T, K)
    return idx, E, R, rank, A


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tables())
def test_layout_properties(tab):
    idx, E, R, rank, A = tab
    T, K = idx.shape
    epr, lo = E // R, rank * (E // R)
    lay = O.layout(idx, E, R, rank, A)
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    assert int(lay["num_invalid"][0]) == int(((flat < -1) | (flat >= E)).sum())
    assert lay["cnt"].tolist() == [int((flat == e).sum()) for e in range(E)]
    member = np.zeros((T, R), np.uint8)
    for t in range(T):
        for e in idx[t]:
            if 0 <= e < E:
                member[t, e // epr] = 1
    assert np.array_equal(lay["in_rank"], member)
    assert lay["ntok_rank"].tolist() == member.sum(axis=0).tolist()
    padded = [-(-int(c) // A) * A for c in lay["cnt"][lo:lo + epr]]
    assert lay["psum"].tolist() == [0] + np.cumsum(padded).tolist()
    local = np.nonzero(valid & (flat >= lo) & (flat < lo + epr))[0]
    order = local[np.argsort(flat[local], kind="stable")]
    expect = []
    for j in range(epr):
        expect += list(range(lay["psum"][j], lay["psum"][j] + int(lay["cnt"][lo + j])))
    assert np.array_equal(lay["slot"].ravel()[order], np.array(expect, np.int64))
    others = np.setdiff1d(np.arange(flat.size), local)
    assert (lay["slot"].ravel()[others] == -1).all()
    for r in range(R):
        toks = np.nonzero(member[:, r])[0]
        col = lay["send_slot"][:, r]
        assert np.array_equal(col[toks], np.arange(len(toks)))
        assert (np.delete(col, toks) == -1).all()


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tables())
def test_dispatch_combine_places_every_entry_once(tab):
    idx, E, R, rank, A = tab
    T, K = idx.shape
    H = 8
    epr, lo = E // R, rank * (E // R)
    # row t of x holds the value t + 1 in every channel (exact in BF16 up to 256)
    x = O.f64_to_bf16(np.repeat(np.arange(1, T + 1, dtype=np.float64)[:, None], H, axis=1)).reshape(T, H)
    lay = O.layout(idx, E, R, rank, A)
    d = O.dispatch(x, idx, None, lay, E, R, rank, A, fp8=False, zero_pad=True)
    out = O.combine(d["recv_x"], lay["slot"], None, None)
    k_local = np.array([int(((idx[t] >= lo) & (idx[t] < lo + epr)).sum()) for t in range(T)], np.float64)
    assert np.array_equal(out, (k_local * np.arange(1, T + 1))[:, None] * np.ones((1, H)))


@st.composite
def received(draw):
    El = draw(st.integers(1, 8))
    N = draw(st.integers(0, 30))
    K = draw(st.integers(1, 5))
    A = draw(st.sampled_from([1, 2, 4, 16]))
    rb = 16 * draw(st.integers(1, 4))
    G = draw(st.integers(0, 3))
    ids = st.one_of(st.integers(0, El - 1), st.just(-1))
    idx = np.array(draw(st.lists(ids, min_size=N * K, max_size=N * K)), np.int64).reshape(N, K)
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return idx, El, A, rb, G, seed


@settings(max_examples=80, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(received())
def test_dispatch_rows_is_a_gather(rec):
    """Receiver placement: every valid row r holds the bytes and scales of the received row that the layout maps
    there (the row's source index, found by brute force over (i, k) with slot[i, k] == r), with that entry's
    weight; padding rows carry -1 / 0 and zeros (zero padding); rows past psum[El] keep the canary."""
    idx, El, A, rb, G, seed = rec
    N, K = idx.shape
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, 256, size=(N, rb), dtype=np.uint8)
    sc = rng.random((N, G), dtype=np.float32) if G else None
    w = rng.random((N, K), dtype=np.float32)
    lay = O.layout(idx, El, 1, 0, A)
    out = O.dispatch_rows(rows, sc, idx, w, lay, El, A, zero_pad=True, recv_fill=(0xA5, -3.0))
    used = int(lay["psum"][-1])
    where = {}
    for i in range(N):
        for k in range(K):
            if lay["slot"][i, k] >= 0:
                where[int(lay["slot"][i, k])] = (i, k)
    for r in range(lay["cap"]):
        if r in where:
            i, k = where[r]
            assert np.array_equal(out["recv_x"][r], rows[i]) and out["recv_src"][r] == i and out["recv_w"][r] == w[i, k]
            if G:
                assert np.array_equal(out["recv_scales"][r], sc[i])
        elif r < used:
            assert (out["recv_x"][r] == 0).all() and out["recv_src"][r] == -1 and out["recv_w"][r] == 0.0
        else:
            assert (out["recv_x"][r] == 0xA5).all() and out["recv_src"][r] == -7


@settings(max_examples=80, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.integers(1, 8), st.integers(0, 20), st.integers(1, 4), st.integers(0, 2 ** 31 - 1), st.booleans(),
       st.booleans())
def test_combine_reduce_sums_what_each_rank_returned(R, T, epr, seed, with_local, with_bias):
    """Source reduce: out[t] = local + sum over the other ranks holding t of their returned row + bias, checked
    against a loop over ranks that locates each token's row in each window by counting the earlier tokens in
    that rank (the send-window definition), independent of the oracle's per-rank token rows."""
    rng = np.random.default_rng(seed)
    E = R * epr
    rank = int(rng.integers(0, R))
    K = min(3, E)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int64) if T else \
        np.zeros((0, K), np.int64)
    H = 8
    lay = O.layout(idx, E, R, rank, 1)
    vals = np.arange(1, 129, dtype=np.float64) / 8.0                 # exact in BF16, small sums exact in fp64
    parts = O.f64_to_bf16(rng.choice(vals, size=(R, T, H)))
    local = O.f64_to_bf16(rng.choice(vals, size=(T, H))) if with_local else None
    bias = O.f64_to_bf16(rng.choice(vals, size=(T, H))) if with_bias else None
    got = O.combine_reduce(parts, lay["send_slot"], rank, local, bias)
    P = O.bf16_to_f32(parts).astype(np.float64)
    for t in range(T):
        ref = np.zeros(H)
        if with_local:
            ref += O.bf16_to_f32(local[t])
        for r in range(R):
            if r == rank or not any(int(e) // epr == r for e in idx[t]):
                continue
            j = sum(1 for u in range(t) if any(int(e) // epr == r for e in idx[u]))
            ref += P[r, j]
        if with_bias:
            ref += O.bf16_to_f32(bias[t])
        assert np.array_equal(got[t], ref)
