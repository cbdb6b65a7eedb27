"""Storage formats: E2M1 codes, E8M0 and E4M3 scales, bfloat16 (oracle, float64).

[MOPD-NVFP4] header paragraph "About NVFP4 quantization": NVFP4 pairs an E2M1
FP4 codebook (magnitudes up to 6, saturating, no NaN/Inf codes) with an FP8
E4M3 scale per 16 elements; MXFP4 instead uses a power-of-two E8M0 scale
([REAP50] "Highlights": ``weight_packed`` U8 + ``weight_scale`` F8_E8M0,
"Model Summary": block = 32).  [GGUF] "Why this model needs an asymmetric
layout": two logical weights share each packed byte.

Readings where the pages are silent (OCP MX conventions): E2M1 bit layout is
sign | 2-bit exponent (bias 1) | 1-bit mantissa; element 2i of a row sits in
the low nibble of byte i; E8M0 byte b means 2^(b-127), 0xFF is NaN; E4M3 is the
"FN" variant (bias 7, subnormals, no infinities, 0x7F/0xFF NaN, max 448).
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes by 3-bit magnitude code, written out from the format
# definition: exponent field e (bias 1), mantissa bit m; e == 0 is subnormal.
def _e2m1_magnitude(code3: int) -> float:
    e, m = (code3 >> 1) & 3, code3 & 1
    if e == 0:
        return 0.5 * m
    return 2.0 ** (e - 1) * (1.0 + 0.5 * m)


E2M1_MAGNITUDES = np.array([_e2m1_magnitude(c) for c in range(8)], dtype=np.float64)


def e2m1_value(nib) -> np.ndarray:
    nib = np.asarray(nib).astype(np.int64)
    mag = E2M1_MAGNITUDES[nib & 7]
    return np.where((nib & 8) != 0, -mag, mag)


def e8m0_value(b) -> np.ndarray:
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def e4m3_value(b) -> np.ndarray:
    b = np.asarray(b).astype(np.int64)
    sign = np.where((b & 0x80) != 0, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m.astype(np.float64), -9)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# Non-negative finite E4M3 values in byte order (bytes 0x00..0x7E), ascending.
_E4M3_POS = e4m3_value(np.arange(0x7F))


def _round_to_table(v: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest table value for v in [table[0], table[-1]];
    an exact midpoint goes to the even index (the even code)."""
    v = np.asarray(v, dtype=np.float64)
    hi = np.searchsorted(table, v, side="left")
    hi = np.clip(hi, 1, len(table) - 1)
    lo = hi - 1
    mid = (table[lo] + table[hi]) * 0.5          # exact: both have few significant bits
    pick_hi = (v > mid) | ((v == mid) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(v <= table[0], 0, idx)
    return idx.astype(np.int64)


def round_to_e4m3(v) -> np.ndarray:
    """Non-negative value -> E4M3 byte, round-to-nearest-even, saturating at 448."""
    v = np.minimum(np.asarray(v, dtype=np.float64), _E4M3_POS[-1])
    return _round_to_table(v, _E4M3_POS).astype(np.uint8)


def round_to_e2m1_magnitude(v) -> np.ndarray:
    """Non-negative value -> 3-bit E2M1 magnitude code, nearest-even, saturating at 6."""
    v = np.minimum(np.asarray(v, dtype=np.float64), E2M1_MAGNITUDES[-1])
    return _round_to_table(v, E2M1_MAGNITUDES).astype(np.uint8)


def bf16_value(bits) -> np.ndarray:
    bits = np.asarray(bits).astype(np.uint32)
    return (bits << 16).view(np.float32).astype(np.float64)


def round_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bfloat16 bit pattern, one rounding (nearest, ties to even).
    Finite values in bfloat16's normal range (the layer never leaves it)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(np.ldexp(m, 8))              # 8 significant bits, half to even
    y = np.ldexp(r, e - 8).astype(np.float32)  # exact: y has <= 9 significant bits
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., k/2] bytes -> [..., k] nibbles; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# value pair of every packed byte: (element 2i = low nibble, element 2i+1 = high nibble)
_PAIR = np.stack([e2m1_value(np.arange(256) & 0xF), e2m1_value(np.arange(256) >> 4)], axis=-1)


def _codes_value(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    return _PAIR[p].reshape(p.shape[:-1] + (p.shape[-1] * 2,))


def dequant_mx(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """MXFP4 [.., n, k/2] codes + [.., n, k/32] E8M0 -> float64 [.., n, k]."""
    v = _codes_value(packed)
    s = e8m0_value(scale)
    return (v.reshape(s.shape + (32,)) * s[..., None]).reshape(v.shape)


def dequant_nv(packed: np.ndarray, scale: np.ndarray, global_scale) -> np.ndarray:
    """NVFP4 [.., n, k/2] codes + [.., n, k/16] E4M3 + global -> float64 [.., n, k]."""
    v = _codes_value(packed)
    s = e4m3_value(scale)
    g = np.asarray(global_scale, dtype=np.float64)
    if g.ndim:
        g = g.reshape(g.shape + (1,) * (s.ndim - g.ndim))
    return (v.reshape(s.shape + (16,)) * (s * g)[..., None]).reshape(v.shape)
