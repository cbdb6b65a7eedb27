"""Exact format identities the scaled-MFMA kernels rely on (CPU, exhaustive).

W4A4 on gfx950's block-scaled MFMA: the instruction takes one E8M0 (power of
two) scale per 32 values of each operand, while an NVFP4 activation value is
c * s * g with an E2M1 code c, an arbitrary E4M3 scale s per 16 values and a
power-of-two global g.  c * s can need 6 significant bits, more than any 8-bit
MFMA operand format holds.  The kernels split it into two E4M3 "planes" that
share one power-of-two scale S = 2^(k-1) g, where s = 2^k (lead + f1/2 +
(2 f2 + f3)/8) (lead = 1 for a normal scale, 0 for a subnormal one, k >= -6):

    hi = c (2 lead + f1),   lo = c (2 f2 + f3) / 4,   c s g = (hi + lo) S.

The pair (hi plane, lo plane) of one 16-value block fills one 32-value block
of an FP8 operand under one E8M0 scale; the FP4 weights of that 16-value block
are fed twice, under their own E8M0 scale.  This file checks, over every E4M3
scale byte and every E2M1 code, with exact rational arithmetic, that hi and lo
are E4M3 values (no rounding anywhere), that they sum back exactly, and that S
is an E8M0 value for the globals in use.
"""
from fractions import Fraction

import numpy as np

import oracle

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e4m3_grid():
    vals = set()
    for b in range(0x7F):                 # 0x7F is NaN
        vals.add(Fraction(oracle.e4m3_value(b).item()))
    return vals


def split(scale_byte: int):
    """(k, lead, f1, f2, f3) of a non-negative E4M3 scale byte."""
    e, m = (scale_byte >> 3) & 15, scale_byte & 7
    lead = 1 if e > 0 else 0
    k = max(e, 1) - 7
    return k, lead, (m >> 2) & 1, (m >> 1) & 1, m & 1


def test_fp8_planes_are_exact_for_every_scale_and_code():
    grid = e4m3_grid()
    checked = 0
    for sb in range(0x7F):
        s = Fraction(oracle.e4m3_value(sb).item())
        k, lead, f1, f2, f3 = split(sb)
        S = Fraction(2) ** (k - 1)
        assert s == Fraction(2) ** k * (lead + Fraction(f1, 2) + Fraction(2 * f2 + f3, 8))
        for code in range(16):
            c = E2M1[code & 7] * (-1 if code & 8 else 1)
            hi = c * (2 * lead + f1)
            lo = c * Fraction(2 * f2 + f3, 4)
            assert abs(hi) in grid and abs(lo) in grid, (sb, code, hi, lo)
            assert (hi + lo) * S == c * s
            checked += 1
    assert checked == 127 * 16


def test_plane_scale_is_e8m0_for_unit_and_power_of_two_globals():
    """S g = 2^(k - 1) g stays inside E8M0's range [2^-127, 2^127] for k in
    [-6, 8] and any global scale 2^j with |j| <= 100."""
    ks = {split(sb)[0] for sb in range(0x7F)}
    assert min(ks) == -6 and max(ks) == 8
    for j in range(-100, 101):
        for k in ks:
            assert -127 <= (k - 1) + j <= 127


def test_plane_values_against_oracle_dequant():
    """The planes of the oracle's own NVFP4 quantisation of random bf16 data
    give back exactly the oracle's NVFP4 values."""
    from synth import random_bf16
    xb = random_bf16(7, (32, 256), std=5.0)
    codes, scales = oracle.quantize_nvfp4(xb, 1.0)
    want = oracle.dequant_nvfp4_act(codes, scales)
    nib = oracle.unpack_codes(codes).astype(np.int64)
    c = oracle.e2m1_value(nib)
    sb = np.repeat(scales.astype(np.int64), 16, axis=-1)
    e, m = (sb >> 3) & 15, sb & 7
    lead = (e > 0).astype(np.int64)
    k = np.maximum(e, 1) - 7
    hi = c * (2 * lead + ((m >> 2) & 1))
    lo = c * (2 * ((m >> 1) & 1) + (m & 1)) / 4.0
    got = (hi + lo) * np.ldexp(1.0, k - 1)
    assert np.array_equal(got, want)


def e2m3_grid():
    """E2M3 (FP6): sign, 2 exponent bits (bias 1), 3 mantissa bits, no specials."""
    vals = set()
    for e in range(4):
        for m in range(8):
            v = Fraction(m, 8) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 8))
            vals.update((v, -v))
    return vals


def test_two_fp6_planes_cannot_hold_every_nvfp4_value():
    """Why the planes are E4M3 and not E2M3 (which the scaled MFMA would run at
    the FP6 rate): for 44 of the 126 non-zero E4M3 scales s there is no power of
    two S for which every c * s / S (c over the E2M1 values) is a sum of two
    E2M3 values, so two FP6 planes under one shared scale cannot be exact."""
    grid = e2m3_grid()
    sums = {a + b for a in grid for b in grid}
    none = []
    for sb in range(1, 0x7F):
        s = Fraction(oracle.e4m3_value(sb).item())
        if not any(all(c * s / Fraction(2) ** a in sums for c in E2M1) for a in range(-40, 40)):
            none.append(sb)
    assert len(none) == 44
    assert 0x7D in none                 # 416 = 2^8 * 1.625
