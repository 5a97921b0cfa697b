"""Pins for the oracle's codecs and byte counts (CPU only).

The oracle's E4M3 and FP4 rules are checked against things other than the
oracle itself:
  * the OCP format anchors and the E2M1 value set (tests/golden/);
  * torch's float8_e4m3fn conversion, an independent library implementation
    of round-to-nearest-even E4M3FN, inside its non-saturating range;
  * a brute-force nearest-value search in exact rational arithmetic
    (fractions.Fraction) with ties to the even code;
  * the constants the pages print (tests/golden/page_constants.json).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from conftest import GOLDEN


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


E2M1 = [float(r[0]) for r in _golden_lines("e2m1_values.txt")]


def _torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ------------------------------------------------------------------ E2M1

def test_e2m1_value_set():
    assert len(E2M1) == 8
    for c in range(16):
        want = E2M1[c & 7] * (-1.0 if c & 8 else 1.0)
        got = O.e2m1_value(c)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), c


# ------------------------------------------------------------------ E4M3

def test_e4m3_anchor_values():
    for code, val in _golden_lines("e4m3_anchors.txt"):
        got = O.e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_e4m3_decode_matches_torch_all_codes():
    ref = _torch_e4m3_table()
    for c in range(256):
        got = O.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], c


def test_e4m3_finite_codes_monotone():
    vals = [O.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert len(vals) == 127 and vals[-1] == 448.0


def _e4m3_inputs(rng):
    table = _torch_e4m3_table()[:0x7F]
    mids = (table[:-1] + table[1:]) / 2          # exact ties between neighbours
    xs = [rng.standard_normal(4000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)]
    xs += [table, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
           rng.uniform(0, 2.0 ** -6, 2000), np.array([0.0, -0.0, 447.9, 448.0, 463.99])]
    x = np.concatenate(xs).astype(np.float32)
    return np.concatenate([x, -x])


def test_e4m3_encode_matches_torch_in_range():
    x = _e4m3_inputs(np.random.default_rng(1))
    x = x[np.abs(x) < 464.0]            # torch does not saturate beyond this
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode_array(x)
    # torch drops the sign of results that round to zero only for +0 inputs
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e4m3_encode_saturates_and_keeps_sign():
    assert O.e4m3_encode(1e9) == 0x7E
    assert O.e4m3_encode(-1e30) == 0xFE
    assert O.e4m3_encode(464.0) == 0x7E
    assert O.e4m3_encode(-0.0) == 0x80
    assert O.e4m3_encode(-1e-30) == 0x80
    assert O.e4m3_encode(2.0 ** -10) == 0x00      # tie to the even code 0
    assert O.e4m3_encode(1.5 * 2.0 ** -9) == 0x02  # tie to the even code 2


# ------------------------------------------------------------------ FP4 groups

def _exact_e4m3(x32: np.float32) -> Fraction:
    """E4M3 RNE of a float32 by brute force over the value table, exact."""
    a = Fraction(float(abs(x32)))
    table = [Fraction(float(v)) for v in _torch_e4m3_table()[:0x7F]]
    best, bd = 0, None
    for c, v in enumerate(table):
        d = abs(a - v)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return table[best]


def _brute_group(x: np.ndarray):
    """Reference FP4 group: scale = E4M3(fp32(amax)/6); codes = nearest of s*E2M1."""
    x = x.astype(np.float32)
    amax = np.max(np.abs(x))
    s_real = np.float32(amax) / np.float32(6.0)          # IEEE fp32 division
    s = _exact_e4m3(s_real)
    grid = [s * Fraction(v) for v in E2M1]
    codes = []
    for xi in x:
        a = Fraction(float(abs(xi)))
        best, bd = 0, None
        for c, g in enumerate(grid):
            d = abs(a - g)
            if bd is None or d < bd or (d == bd and c % 2 == 0):
                best, bd = c, d
        if s == 0:
            best = 0
        codes.append(best | (8 if np.signbit(xi) else 0))
    return np.array(codes, np.uint8), s


def _groups(rng):
    gs = [rng.standard_normal(16) * sc for sc in (1.0, 8.0, 0.01, 1e-4, 300.0)]
    gs.append(np.zeros(16))
    gs.append(-np.zeros(16))
    gs.append(np.r_[rng.standard_normal(15) * 1e-9, 3000.0])   # scale saturates at 448
    gs.append(np.r_[rng.standard_normal(15) * 1e-3, 1e-3])
    gs.append(np.full(16, 6e-4))                                 # scale rounds to 0
    # exact midpoints s*t_j: amax = 6 -> s = 1; entries at the rounding thresholds
    gs.append(np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                        -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 0.0]))
    gs.append(np.array([12.0, 0.5, 1.5, 2.5, 3.5, 5.0, 7.0, 10.0,
                        0.49, 1.51, 2.49, 3.51, 4.99, 7.01, 9.99, 11.9]))
    # amax/6 not representable: s rounds down, so amax lies above 6*s (saturates)
    gs.append(np.r_[6.4, rng.uniform(-6.4, 6.4, 15)])
    return [g.astype(np.float32) for g in gs]


def test_fp4_group_matches_exact_brute_force():
    rng = np.random.default_rng(7)
    groups = _groups(rng) + [rng.standard_normal(16).astype(np.float32) * rng.uniform(0.01, 40)
                             for _ in range(400)]
    for g in groups:
        nib, sc = O.fp4_group(g)
        want, s = _brute_group(g)
        assert Fraction(O.e4m3_value(sc)) == s, g
        assert np.array_equal(nib, want), (g, nib, want)


def test_fp4_error_bound_when_not_saturated():
    """|x - s*q(x/s)| <= s at the top of the grid, <= s/4 below 2 (grid step / 2)."""
    rng = np.random.default_rng(3)
    for _ in range(300):
        g = (rng.standard_normal(16) * rng.uniform(0.1, 20)).astype(np.float32)
        nib, sc = O.fp4_group(g)
        s = O.e4m3_value(sc)
        for xi, c in zip(g, nib):
            v = O.e2m1_value(int(c)) * s
            if abs(xi) <= 6 * s:
                half_step = s * (0.25 if abs(xi) <= 2 * s else 0.5 if abs(xi) <= 4 * s else 1.0)
                assert abs(float(xi) - v) <= half_step + 1e-12


# ------------------------------------------------------------------ byte counts

def test_byte_counts_against_pages():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        pc = json.load(f)
    D, G = 128, pc["channels_per_fp4_scale"]["value"]
    per_vec = D * pc["fp4_bytes_per_element"]["value"] + D // G   # codes + E4M3 scales
    assert per_vec == 72
    assert O.record_bytes() == 2 * per_vec == 144
    # FP4 + per-16 scale against one FP8 byte per channel: 9/16, about half
    assert per_vec / (D * 1.0) == pytest.approx(9 / 16)
    assert abs(per_vec / D - pc["fp4_vs_fp8_capacity"]["value"]) < 0.1
    assert pc["fp4_bytes_per_element"]["value"] / pc["fp16_bytes_per_element"]["value"] == 0.25
    assert pc["pool_blocks"]["value"] * pc["block_positions"]["value"] == pc["pool_positions"]["value"]
