"""Compact MXFP4 expert storage, 4.125 bits per weight (oracle).

[PRO6000] "What makes it fast" (speed v4, from earlier releases): a lossless
compact encoding of the experts, "nvfp4c", 4.125 instead of 4.5 bits per
weight with the same values.  The page gives the size and the losslessness,
not the layout; parity unpinned as to the layout -- the one below is this
library's reading, chosen as the plainest that reaches 4.125 bits exactly:

  * the E2M1 codes stay as they are (4 bits per weight);
  * each 32-value block keeps a 4-bit exponent code c in 0..15 instead of its
    8-bit E8M0 scale (4 / 32 = 0.125 bits per weight); block 2i is the low
    nibble of byte i;
  * each matrix keeps one power-of-two base 2^b with b = (largest finite block
    exponent) - 15, and a block's scale is 2^(b + c).

Blocks whose exponent lies below b cannot be expressed: an all-zero block
(every code +-0) gets c = 0 and is counted "zero_oor" (exact: its values are
0); any other is clamped to c = 0 and counted "rerounded" (not exact).  An
E8M0 NaN scale (0xFF) has no code: c = 15, counted "nan".  A matrix with no
finite block gets b = 0.  The encoding is lossless exactly when both the
rerounded and nan counts are zero; the values are then those of the MXFP4
tensors (pinned: dequant_compact == dequant_mx).
"""
from __future__ import annotations

import numpy as np

from .formats import _codes_value, unpack_codes

SPAN = 15


def compact_mx(mx_scale: np.ndarray, packed: np.ndarray):
    """mx_scale u8 [M, n, k/32], packed u8 [M, n, k/2] ->
    (exponent codes u8 [M, n, k/64], base f32 [M] (= 2^b), counters dict)."""
    mx_scale = np.asarray(mx_scale, dtype=np.uint8)
    M = mx_scale.shape[0]
    out = np.empty(mx_scale.shape[:-1] + (mx_scale.shape[-1] // 2,), np.uint8)
    base = np.empty(M, np.float32)
    cnt = {"blocks": 0, "zero_oor": 0, "rerounded": 0, "nan": 0}
    for m in range(M):
        sb = mx_scale[m].astype(np.int64)
        is_nan = sb == 255
        e = sb - 127
        finite = e[~is_nan]
        b = int(finite.max()) - SPAN if finite.size else 0
        c = e - b
        low = (~is_nan) & (c < 0)
        if low.any():
            nib = unpack_codes(packed[m]).reshape(sb.shape + (32,))
            all_zero = np.all((nib & 7) == 0, axis=-1)
            cnt["zero_oor"] += int((low & all_zero).sum())
            cnt["rerounded"] += int((low & ~all_zero).sum())
        c = np.where(is_nan, SPAN, np.clip(c, 0, SPAN))
        cnt["nan"] += int(is_nan.sum())
        cnt["blocks"] += int(sb.size)
        out[m] = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
        base[m] = np.float32(np.ldexp(1.0, b))
    return out, base, cnt


def dequant_compact(packed: np.ndarray, codes4: np.ndarray, base) -> np.ndarray:
    """Compact [.., n, k/2] codes + [.., n, k/64] exponent codes + base -> float64 [.., n, k]."""
    v = _codes_value(packed)
    c = unpack_codes(codes4).astype(np.int64)                 # one exponent code per 32-value block
    s = np.ldexp(np.asarray(base, np.float64).reshape(np.shape(base) + (1,) * (c.ndim - np.ndim(base))), c)
    return (v.reshape(c.shape + (32,)) * s[..., None]).reshape(v.shape)
