"""NVFP4 activation quantisation with a per-layer global scale (oracle).

[MOPD-NVFP4] "About NVFP4 quantization": E2M1 codes with an E4M3 scale over
16-element micro-blocks, saturating rather than overflowing.  "Quantization
Details": one activation global scale per layer, shipped as 1.0 (the "unit
scale"); the capped calibration variant caps the down-projection input at 2688.

Reading adopted for the step the pages leave open: per row and per 16
consecutive values of the bfloat16 input, a = max|x|, the block scale is
s = E4M3(a / (6 * g)) rounded to nearest-even and saturated at 448 (g = the
global "input scale", a power of two; 1.0 here); codes q = E2M1(x / (s * g)),
nearest-even, saturated at 6, carrying the sign of x (so -0 for a negative
value that rounds to zero).  A block whose scale rounds to 0 gets +0 codes.
The value the GEMM consumes is q * s * g.  With g = 1 every |x| >= 2688 = 6 x 448
saturates to +-2688.  The "error-minimising scale selection" the card mentions
is not specified and is not built.
"""
from __future__ import annotations

import numpy as np

from .formats import (bf16_value, e2m1_value, e4m3_value, e8m0_value, round_to_e2m1_magnitude,
                      round_to_e4m3, unpack_codes)


def quantize_nvfp4(x_bits: np.ndarray, input_scale: float = 1.0):
    """bf16 bits [rows, k] -> (codes u8 [rows, k/2], scales u8 [rows, k/16])."""
    x = bf16_value(x_bits)
    rows, k = x.shape
    xb = x.reshape(rows, k // 16, 16)
    amax = np.abs(xb).max(axis=-1)
    g = float(input_scale)
    s_byte = round_to_e4m3(amax / (6.0 * g))
    s = e4m3_value(s_byte)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.abs(xb) / (s[..., None] * g)
    mag = round_to_e2m1_magnitude(np.where(s[..., None] > 0, r, 0.0))
    neg = np.signbit(xb) & (s[..., None] > 0)
    nib = (mag | np.where(neg, 8, 0)).astype(np.uint8).reshape(rows, k)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, s_byte


def dequant_nvfp4_act(codes: np.ndarray, scales: np.ndarray, input_scale: float = 1.0) -> np.ndarray:
    v = e2m1_value(unpack_codes(codes))
    s = np.repeat(e4m3_value(scales), 16, axis=-1)
    return v * s * float(input_scale)


# ------------------------------------------------------------------ MXFP8
# [PRO6000] "Quantization, context and quality", Activations: prompt batches
# run the expert GEMMs on E4M3 activations with a power-of-two scale per 32
# values (MXFP8); "What makes it fast" (speed v5.2): FP8 x FP4 block-scaled
# GEMMs for the experts, on the stored weights as they are.
#
# Reading adopted for the scale (the pages name the format, not the rule): the
# OCP Microscaling definition of MXFP8 E4M3.  Per row and 32 consecutive values
# of the bfloat16 input, the shared scale is X = 2^(floor(log2 max|x|) - 8)
# (8 = the exponent of E4M3's largest power of two), clamped to E8M0's range
# [2^-127, 2^127]; each element is x / X rounded to nearest-even E4M3
# (subnormals included) and saturated at +-448, keeping the sign of x.  A
# block of zeros gets X = 2^-127 and zero codes.  With this rule max|x| / X lies
# in [256, 512), so the largest elements of a block can saturate at 448 * X.
E8M0_BIAS = 127


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for finite a > 0, exactly (frexp: a = m 2^e, 0.5 <= m < 1)."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


def quantize_mxfp8(x_bits: np.ndarray):
    """bf16 bits [rows, k] -> (E4M3 codes u8 [rows, k], E8M0 scales u8 [rows, k/32])."""
    x = bf16_value(x_bits)
    rows, k = x.shape
    xb = x.reshape(rows, k // 32, 32)
    amax = np.abs(xb).max(axis=-1)
    exp = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - 8, -E8M0_BIAS)
    exp = np.clip(exp, -E8M0_BIAS, E8M0_BIAS)
    scale_byte = (exp + E8M0_BIAS).astype(np.uint8)
    r = np.abs(xb) / np.ldexp(1.0, exp)[..., None]          # exact: a power-of-two division
    mag = round_to_e4m3(r)                                   # nearest-even, saturating at 448
    sign = np.where(np.signbit(xb), 0x80, 0).astype(np.uint8)
    return (mag | sign).reshape(rows, k).astype(np.uint8), scale_byte


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3 codes [rows, k] + E8M0 scales [rows, k/32] -> float64 values."""
    v = e4m3_value(codes)
    s = np.repeat(e8m0_value(scales), 32, axis=-1)
    return v * s
