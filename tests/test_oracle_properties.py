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
