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

from .formats import (bf16_value, e2m1_value, e4m3_value, round_to_e2m1_magnitude,
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
