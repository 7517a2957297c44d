"""Pins for the oracle's layout: the pages' padding worked example, a hand-traced table, brute-force counts,
numpy's stable argsort for the expert-major permutation, and invariants on every workload."""
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_padding_worked_example():
    """MoE-comm page, section 三 (padding): counts 1/1/126 at alignment 128 -> 384 slots, A_pad = 3."""
    g = json.load(open(os.path.join(GOLD, "padding_worked_example.json")))
    idx = np.concatenate([np.full(c, e, np.int64) for e, c in enumerate(g["counts"])]).reshape(-1, 1)
    lay = O.layout(idx, num_experts=len(g["counts"]), expert_alignment=g["expert_alignment"])
    assert list(lay["psum"]) == g["expected_psum"]
    assert lay["psum"][-1] == g["expected_slots"]
    valid = int((lay["row_src"][: lay["psum"][-1]] >= 0).sum())
    assert valid == g["expected_valid_rows"]
    assert lay["psum"][-1] / valid == g["expected_A_pad"]


def test_hand_traced_layout():
    g = json.load(open(os.path.join(GOLD, "layout_tiny.json")))
    lay = O.layout(np.array(g["topk_idx"], np.int64), g["num_experts"], g["num_ranks"], g["rank"],
                   g["expert_alignment"])
    assert lay["cap"] == g["cap"]
    assert lay["cnt"].tolist() == g["cnt"]
    assert lay["ntok_rank"].tolist() == g["ntok_rank"]
    assert lay["in_rank"].tolist() == g["in_rank"]
    assert lay["psum"].tolist() == g["psum"]
    assert lay["slot"].tolist() == g["slot"]
    n = len(g["row_src_first_rows"])
    assert lay["row_src"][:n].tolist() == g["row_src_first_rows"]
    assert (lay["row_src"][n:] == -1).all()
    assert lay["send_slot"].tolist() == g["send_slot"]
    assert int(lay["num_invalid"][0]) == g["num_invalid"]


def _brute_layout_checks(idx, E, R, rank, A, lay):
    T, K = idx.shape
    epr = E // R
    lo = rank * epr
    # counts by brute force
    for e in range(E):
        assert lay["cnt"][e] == int((idx == e).sum())
    # membership and per-rank counts by brute force over tokens
    for t in range(T):
        ranks = {int(e) // epr for e in idx[t] if 0 <= e < E}
        assert set(np.nonzero(lay["in_rank"][t])[0].tolist()) == ranks
    assert lay["ntok_rank"].tolist() == [int(lay["in_rank"][:, r].sum()) for r in range(R)]
    # psum: aligned, closed form from counts
    loc = lay["cnt"][lo: lo + epr]
    padded = -(-loc // A) * A
    assert lay["psum"].tolist() == [0] + np.cumsum(padded).tolist()
    assert all(p % A == 0 for p in lay["psum"])
    assert lay["psum"][-1] <= lay["cap"]
    # permutation == numpy stable argsort of local entries by expert
    flat = idx.ravel()
    local = np.nonzero((flat >= lo) & (flat < lo + epr))[0]
    order = local[np.argsort(flat[local], kind="stable")]
    rows = []
    for e in range(epr):
        rows.extend(range(lay["psum"][e], lay["psum"][e] + loc[e]))
    slot = lay["slot"].ravel()
    assert np.array_equal(slot[order], np.array(rows, np.int64))
    assert (slot[np.setdiff1d(np.arange(flat.size), local)] == -1).all()
    # row_src is the inverse map; every other row is -1
    rs = lay["row_src"]
    assert np.array_equal(rs[slot[order]], order // K)
    mask = np.ones(lay["cap"], bool)
    mask[slot[order]] = False
    assert (rs[mask] == -1).all()
    # per-rank token rows: dense, ascending token order (own rank: token-major receive rows)
    for r in range(R):
        col = lay["send_slot"][:, r]
        toks = np.nonzero(lay["in_rank"][:, r])[0]
        assert np.array_equal(col[toks], np.arange(len(toks)))
        assert (np.delete(col, toks) == -1).all()


@pytest.mark.parametrize("T,K,E,R,rank,A,seed", [
    (1, 1, 1, 1, 0, 1, 0), (5, 3, 7, 1, 0, 4, 1), (37, 4, 16, 4, 2, 8, 2), (64, 8, 32, 8, 7, 3, 3),
    (130, 6, 24, 3, 1, 16, 4), (97, 2, 10, 5, 4, 1, 5)])
def test_random_tables_brute_force(T, K, E, R, rank, A, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, K)).astype(np.int64)   # duplicates within a token allowed
    lay = O.layout(idx, E, R, rank, A)
    _brute_layout_checks(idx, E, R, rank, A, lay)
    assert int(lay["num_invalid"][0]) == 0


def test_unused_and_invalid_entries():
    idx = np.array([[0, -1], [5, 2], [-3, 1], [99, -1]], np.int64)
    lay = O.layout(idx, num_experts=4, expert_alignment=2)
    assert int(lay["num_invalid"][0]) == 3         # 5, -3, 99 are dropped; -1 is just unused
    assert lay["cnt"].tolist() == [1, 1, 1, 0]
    assert lay["slot"].tolist() == [[0, -1], [-1, 4], [-1, 2], [-1, -1]]
    assert lay["psum"].tolist() == [0, 2, 4, 6, 6]


def test_empty_inputs():
    lay = O.layout(np.zeros((0, 4), np.int64), num_experts=8, expert_alignment=16)
    assert lay["psum"].tolist() == [0] * 9
    assert lay["cnt"].tolist() == [0] * 8
    assert lay["cap"] == 8 * 15
    assert (lay["row_src"] == -1).all()


@pytest.mark.parametrize("name", W.ORDER)
def test_workload_invariants(name):
    inp = W.make_inputs(name)
    c = inp["cfg"]
    idx = inp["topk_idx"].numpy()
    lay = O.layout(idx, c.num_experts, c.num_ranks, c.rank, c.expert_alignment)
    T, K = idx.shape
    assert lay["cnt"].sum() == T * K                      # no -1 entries in the workloads
    assert lay["cap"] == T * K + (c.num_experts // c.num_ranks) * (c.expert_alignment - 1)
    assert lay["ntok_rank"].sum() == sum(len({int(e) // (c.num_experts // c.num_ranks) for e in row})
                                         for row in idx)
    if c.num_ranks == 1:
        assert (lay["in_rank"] == 1).all()
    if T <= 256:
        _brute_layout_checks(idx, c.num_experts, c.num_ranks, c.rank, c.expert_alignment, lay)
