"""Pins for the oracle's number formats: OCP e4m3fn and BF16.

Each codec is checked against (a) hand-worked codes from the format definition (tests/golden/e4m3_codes.json),
(b) brute-force nearest-value search over the whole code table, ties to the even code, and (c) torch's CPU
casts, which are independent library routines.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _all_e4m3_values():
    """Decoded value of every code, from the bit-field definition written independently here."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = m * 2.0 ** -9
        else:
            vals[c] = (1 + m / 8) * 2.0 ** (e - 7)
        if s:
            vals[c] = -vals[c]
    return vals


def _brute_e4m3(v):
    """Nearest finite code by exhaustive search; ties to the even code; beyond 448 saturate."""
    table = _all_e4m3_values()
    finite = [c for c in range(256) if not np.isnan(table[c])]
    out = np.empty(len(v), np.uint8)
    for i, x in enumerate(np.asarray(v, np.float64)):
        if abs(x) > 448.0:
            out[i] = 0x7E | (0x80 if x < 0 else 0)
            continue
        best, bestd = None, None
        for c in finite:
            if (table[c] == 0.0) and (np.signbit(table[c]) != np.signbit(x)):
                continue  # zero carries the sign of the input
            d = abs(table[c] - x)
            if bestd is None or d < bestd or (d == bestd and (c & 1) == 0 and (best & 1) == 1):
                best, bestd = c, d
        out[i] = best
    return out


def test_e4m3_golden_codes():
    cases = json.load(open(os.path.join(GOLD, "e4m3_codes.json")))["cases"]
    v = np.array([c["value"] for c in cases], np.float32)
    got = O.e4m3_encode(v)
    for c, g in zip(cases, got):
        assert int(g) == c["code"], (c, int(g))


def test_e4m3_decode_matches_definition_and_torch():
    table = _all_e4m3_values()
    dec = O.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    assert np.array_equal(np.isnan(dec), np.isnan(table))
    ok = ~np.isnan(table)
    assert np.array_equal(dec[ok], table[ok])
    assert np.array_equal(np.signbit(dec[ok]), np.signbit(table[ok]))
    tdec = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(tdec), np.isnan(table))
    assert np.array_equal(tdec[ok], dec[ok])


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    again = O.e4m3_encode(O.e4m3_decode(codes))
    assert np.array_equal(again, codes)


def _probe_values():
    """Every code value, every midpoint between neighbours, and the float32 neighbours of those."""
    table = _all_e4m3_values()
    pos = np.unique(table[(~np.isnan(table)) & (table >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids, [448.0, 455.9, 464.0, 470.0, 1e4, 3e38]]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(0))
    v = np.concatenate([base, up, dn]).astype(np.float32)
    return np.concatenate([v, -v])


def test_e4m3_encode_vs_brute_force():
    v = _probe_values()
    rng = np.random.default_rng(7)
    r = (rng.standard_normal(4000) * np.exp(rng.uniform(-12, 7, 4000))).astype(np.float32)
    v = np.concatenate([v, r])
    assert np.array_equal(O.e4m3_encode(v), _brute_e4m3(v))


def test_e4m3_encode_vs_torch_cast_in_range():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        _probe_values(),
        (rng.standard_normal(200000) * np.exp(rng.uniform(-14, 6.1, 200000))).astype(np.float32),
        rng.uniform(-448, 448, 100000).astype(np.float32)])
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v), ref)


def test_e4m3_saturates_instead_of_nan():
    v = np.array([449.0, 463.99, 464.0, 480.0, 1e6, np.inf, -449.0, -np.inf], np.float32)
    got = O.e4m3_encode(v)
    assert list(got) == [0x7E] * 6 + [0xFE] * 2
    assert O.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_bf16_from_float32_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # ties: float32 values exactly halfway between two bf16 neighbours
    ties = ((rng.integers(0, 2 ** 16, 20000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    v = np.concatenate([v, ties, np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38, 1e-45], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_from_double_brute_force():
    """Doubles that are not float32 values: nearest BF16 by checking the two neighbours, ties to even."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))
    got = O.f64_to_bf16(v)
    for x, g in zip(v, got):
        lo_bits = (np.array([x], np.float32).view(np.uint32)[0] >> 16)  # truncation toward zero (|x| small)
        cands = [int(lo_bits) - 1, int(lo_bits), int(lo_bits) + 1, int(lo_bits) + 2]
        vals = [float((np.array([c], np.uint32) << 16).view(np.float32)[0]) for c in cands]
        d = [abs(a - x) for a in vals]
        m = min(d)
        best = [c for c, dd in zip(cands, d) if dd == m]
        pick = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        assert int(g) == pick, (x, int(g), pick)


def test_bf16_special_values():
    v = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e300, -1e300], np.float64)
    got = O.f64_to_bf16(v)
    assert list(got) == [0x7FC0, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x7F80, 0xFF80]
