"""Pins of the oracle's number formats against things other than itself:
torch's own float8_e4m3fn and bfloat16 conversions (independent library
routines), the published format tables under tests/golden/, and brute-force
nearest-value searches."""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3_encode(v):
    t = torch.from_numpy(np.asarray(v, np.float32).copy())
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _load(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                rows.append((int(a, 0), float(b)))
    return rows


# --- bf16 -------------------------------------------------------------------

def test_bf16_roundtrip_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(50000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38], np.float32),
    ])
    # values sitting exactly on a bf16 rounding midpoint (ties)
    u = rng.integers(0, 2**16, 5000, dtype=np.uint32) << np.uint32(16)
    ties = (u | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    v = np.concatenate([v, ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(v), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_to_f32(ref).view(np.uint32), back.view(np.uint32))


# --- E4M3 -------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    mine = oracle.e4m3_decode_table()
    ref = _torch_e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # signed zeros
    assert np.signbit(mine[0x80]) and not np.signbit(mine[0x00])


def test_e4m3_golden_anchors():
    t = oracle.e4m3_decode_table()
    for code, val in _load("e4m3_anchors.txt"):
        if np.isnan(val):
            assert np.isnan(t[code])
        else:
            assert t[code] == val and np.signbit(t[code]) == np.signbit(val)


def test_e4m3_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_encode_midpoints_and_neighbours_match_torch():
    pos = oracle.e4m3_decode(np.arange(0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    v = np.concatenate([mids, up, dn, -mids, -up, -dn])
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3_encode(v))


def test_e4m3_encode_random_matches_torch_in_range():
    rng = np.random.default_rng(1)
    parts = []
    for e in range(-14, 9):
        parts.append((rng.uniform(-1, 1, 40000) * 2.0 ** e).astype(np.float32))
    v = np.concatenate(parts + [np.array([0.0, -0.0, 464.0, -464.0], np.float32)])
    v = v[np.abs(v) <= 464.0]  # torch turns values above 464 into NaN
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3_encode(v))


def test_e4m3_encode_brute_force_nearest():
    """Nearest value by exhaustive search over the 254 finite codes, ties to
    the even code, saturation above 448."""
    table = oracle.e4m3_decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(table[c])])
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(3000) * 40, rng.standard_normal(500) * 0.01,
                        np.array([500.0, -1e9, 448.0, 470.0], )]).astype(np.float32)
    got = oracle.e4m3_encode(v)
    for x, c in zip(v.astype(np.float64), got):
        xs = min(max(x, -448.0), 448.0)
        d = np.abs(table[finite] - xs)
        best = finite[d == d.min()]
        # among equal distances keep same-sign code, then the even mantissa
        best = [b for b in best if (b >= 0x80) == (np.signbit(x))] or list(best)
        if len(best) > 1:
            best = [b for b in best if b % 2 == 0]
        assert c == best[0], (x, c, best)


def test_e4m3_encode_saturates_and_keeps_sign():
    v = np.array([448.0, 464.0, 465.0, 1e6, -465.0, -3e38, -0.0, 0.0], np.float32)
    assert list(oracle.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x00]
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([np.nan], np.float32))


# --- E2M1 and the fold --------------------------------------------------------

def test_e2m1_table_matches_published_values():
    t = oracle.e2m1_decode_table()
    for code, val in _load("e2m1_values.txt"):
        assert t[code] == val and np.signbit(t[code]) == np.signbit(val)


def test_e2m1_encode_brute_force():
    t = oracle.e2m1_decode_table()
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-8, 8, 20000),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.25, 7.0])]
                       ).astype(np.float32)
    got = oracle.e2m1_encode(v)
    for x, c in zip(v.astype(np.float64), got):
        xs = min(max(x, -6.0), 6.0)
        cands = [k for k in range(16) if (k >= 8) == (x < 0)]
        d = np.array([abs(t[k] - xs) for k in cands])
        best = [cands[i] for i in np.nonzero(d == d.min())[0]]
        if len(best) > 1:
            best = [b for b in best if b % 2 == 0]
        assert c == best[0], (x, c, best)


def test_fold_table_is_nearest_e4m3_of_exact_product():
    """T[c][b] decodes to the E4M3 value nearest to e2m1(c)*e4m3(b)/8, ties
    to the even code, for all 16 x 256 pairs; the NaN scales give NaN."""
    T = oracle.fold_table()
    e2 = oracle.e2m1_decode_table()
    e4 = _torch_e4m3_decode(np.arange(256))
    finite = [c for c in range(256) if not np.isnan(e4[c])]
    fv = e4[finite]
    for c in range(16):
        for b in range(256):
            if np.isnan(e4[b]):
                assert np.isnan(e4[T[c, b]])
                continue
            p = e2[c] * e4[b] / 8.0  # exact in float64
            assert abs(p) <= 336.0
            d = np.abs(fv - p)
            best = [finite[i] for i in np.nonzero(d == d.min())[0]]
            neg = np.signbit(p)
            best = [x for x in best if (x >= 0x80) == neg] or best
            if len(best) > 1:
                best = [x for x in best if x % 2 == 0]
            assert T[c, b] == best[0], (c, b, T[c, b], best)


def test_fold_table_exact_when_product_has_few_bits():
    T = oracle.fold_table()
    e2 = oracle.e2m1_decode_table()
    e4 = _torch_e4m3_decode(np.arange(256))
    n_exact = 0
    for c in range(16):
        for b in range(0x08, 0x7F):  # normal, positive scales
            p = e2[c] * e4[b] / 8.0
            m, _ = np.frexp(abs(p))
            if p != 0 and abs(p) >= 2.0 ** -6 and (m * 16) == np.floor(m * 16):
                assert e4[T[c, b]] == p
                n_exact += 1
    assert n_exact > 1000
