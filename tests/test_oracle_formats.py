"""Pins for the oracle's format codecs (CPU only).

Each check compares the oracle against something other than itself: the
pages' printed values (golden files), torch's own float8 codecs, or exact
rational brute force.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_numbers(name):
    vals = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                vals.extend(float(v) for v in line.split())
    return vals


def test_e2m1_table_matches_pages():
    table = _read_numbers("e2m1_magnitudes.txt")
    assert len(table) == 8 and max(table) == 6.0
    v = oracle.e2m1_value(np.arange(16))
    assert list(v[:8]) == table
    assert list(-v[8:]) == table
    assert np.signbit(v[8])          # code 0b1000 is -0


def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e8m0_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_value(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    # torch stores 2^-127 as a float32 subnormal; compare as float64 powers of two
    assert np.array_equal(got[:255], np.ldexp(1.0, np.arange(255) - 127))
    assert np.array_equal(ref[1:255], got[1:255])


def test_round_to_e4m3_matches_torch_rne():
    rng = np.random.default_rng(0)
    pos = oracle.e4m3_value(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([
        pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.uniform(0, 448, 20000), np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448), 20000)),
    ]).astype(np.float32)        # torch converts from float32; all chosen values are exact there
    vals = np.clip(vals, 0, 448).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.round_to_e4m3(vals.astype(np.float64))
    assert np.array_equal(ref, got)


def test_round_to_e4m3_saturates():
    got = oracle.round_to_e4m3(np.array([448.0, 460.0, 500.0, 1e9]))
    assert list(got) == [0x7E] * 4


def _nearest_even_fraction(x: Fraction, table):
    best = None
    for i, t in enumerate(table):
        d = abs(x - Fraction(t))
        key = (d, i % 2)            # smaller distance first, then the even code
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def test_round_to_e2m1_brute_force():
    table = _read_numbers("e2m1_magnitudes.txt")
    rng = np.random.default_rng(1)
    mids = [(a + b) / 2 for a, b in zip(table[:-1], table[1:])]
    vals = list(table) + mids + list(rng.uniform(0, 6, 3000)) + [6.0, 7.0, 100.0]
    got = oracle.round_to_e2m1_magnitude(np.array(vals))
    for v, g in zip(vals, got):
        exp = 7 if v >= 6 else _nearest_even_fraction(Fraction(v), table)
        assert g == exp, (v, g, exp)


def test_round_to_bf16_brute_force():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                        [0.0, -0.0, 1.0, -2.5, 3.0e5]])
    # exact bf16 midpoints and their neighbours (double rounding through float32 would fail these)
    b = oracle.bf16_value(np.array([0x3F80, 0x4049, 0xC2AB], np.uint16))
    ulp = b * 2.0 ** -7
    x = np.concatenate([x, b + ulp / 2, b + ulp / 2 + ulp * 2.0 ** -30, b + ulp / 2 - ulp * 2.0 ** -30,
                        b + 1.5 * ulp])
    got = oracle.round_to_bf16_bits(x)
    # float32-exact inputs: torch's float32 -> bfloat16 conversion is round-nearest-even
    f32_exact = x.astype(np.float32).astype(np.float64) == x
    ref = torch.from_numpy(x[f32_exact].astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[f32_exact], ref)
    # everything: exact rational check against the two neighbouring bf16 values
    for xi, gi in zip(x, got):
        v = Fraction(float(oracle.bf16_value(np.uint16(gi))))
        xf = Fraction(float(xi))
        if v == 0:
            assert xf == 0
            continue
        # neighbours of v
        lo = Fraction(float(oracle.bf16_value(np.uint16(gi - 1)))) if (gi & 0x7FFF) else -v
        hi = Fraction(float(oracle.bf16_value(np.uint16(gi + 1))))
        assert abs(xf - v) <= abs(xf - lo) and abs(xf - v) <= abs(xf - hi), (xi, gi)
        if abs(xf - v) == abs(xf - lo) or abs(xf - v) == abs(xf - hi):
            assert gi % 2 == 0, (xi, gi)


def test_dequant_mx_elementwise():
    from synth import random_mx_small
    packed, scale = random_mx_small(3, 2, 8, 64, lo=100, hi=140)
    table = _read_numbers("e2m1_magnitudes.txt")
    got = oracle.dequant_mx(packed, scale)
    for e in range(2):
        for n in range(8):
            for k in range(64):
                byte = int(packed[e, n, k // 2])
                nib = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
                v = table[nib & 7] * (-1 if nib & 8 else 1) * 2.0 ** (int(scale[e, n, k // 32]) - 127)
                assert got[e, n, k] == v


def test_dequant_nv_uses_global():
    codes = np.array([[0x21, 0x7F, 0x00, 0x8A, 0x11, 0x22, 0x33, 0x44]], np.uint8)   # k = 16
    sc = np.array([[0x38]], np.uint8)           # E4M3 1.0
    v1 = oracle.dequant_nv(codes, sc, 1.0)
    v2 = oracle.dequant_nv(codes, sc, 0.25)
    assert np.array_equal(v1 * 0.25, v2)
    # byte 0x21: low nibble 1 (0.5) then 2 (1.0); byte 0x7F: 0xF (-6) then 7 (6)
    assert list(v1[0, :4]) == [0.5, 1.0, -6.0, 6.0]
