"""Exact MXFP4 -> NVFP4 weight transcode (oracle).

[MOPD-NVFP4] header: every E2M1 code is kept byte for byte and each E8M0 block
scale is re-expressed exactly as two E4M3 block scales; "Reproduce the
checkpoint" reports counts of blocks, all-zero blocks and out-of-E4M3-range
("re-rounded") blocks.  [RL-NVFP4] "What changed": each E8M0 scale for 32
weights becomes two E4M3 scales for 16 weights combined with an exact
power-of-two global scale; all scale groups were representable.

Reading adopted (parity unpinned -- the pages do not fix which exact global
scale they chose, and many are exact): one global scale per matrix,
G = (largest finite block exponent of the matrix) - 8, so the largest block
scale maps to 2^8 = 256, the largest E4M3 power of two.  A block with exponent
e then needs the E4M3 power of two 2^(e-G); exponents down to 2^-9 (E4M3
subnormals) are representable.  Blocks below that range are written as zero and
counted "all-zero" if all 32 codes are +-0, else clamped to 2^-9 and counted
"re-rounded".  E8M0 NaN (0xFF) becomes E4M3 NaN (0x7F) and is counted.  A matrix
with no finite block gets G = 0.
"""
from __future__ import annotations

import numpy as np

from .formats import unpack_codes


def _e4m3_pow2_byte(k: np.ndarray) -> np.ndarray:
    """E4M3 byte of 2^k for -9 <= k <= 8."""
    k = np.asarray(k, dtype=np.int64)
    normal = (k + 7) << 3                   # exponent field k+7, mantissa 0
    sub = np.left_shift(1, np.clip(k + 9, 0, 2))   # 2^k = M * 2^-9 with M = 2^(k+9)
    return np.where(k >= -6, normal, sub).astype(np.uint8)


def transcode_mx_to_nv(mx_scale: np.ndarray, packed: np.ndarray):
    """mx_scale u8 [M, n, k/32], packed u8 [M, n, k/2] ->
    (nv_scale u8 [M, n, k/16], global_scale f32 [M], counters dict)."""
    mx_scale = np.asarray(mx_scale, dtype=np.uint8)
    M = mx_scale.shape[0]
    nv = np.empty(mx_scale.shape[:-1] + (mx_scale.shape[-1] * 2,), np.uint8)
    glob = np.empty(M, np.float32)
    cnt = {"blocks": 0, "zero_oor": 0, "rerounded": 0, "nan": 0}
    for m in range(M):
        b = mx_scale[m].astype(np.int64)
        is_nan = b == 255
        e = b - 127
        finite = e[~is_nan]
        G = int(finite.max()) - 8 if finite.size else 0
        k = e - G
        byte = _e4m3_pow2_byte(np.clip(k, -9, 8))
        oor = (~is_nan) & (k < -9)
        if oor.any():
            nib = unpack_codes(packed[m]).reshape(b.shape + (32,))
            all_zero = np.all((nib & 7) == 0, axis=-1)
            z = oor & all_zero
            byte = np.where(z, np.uint8(0), byte)
            cnt["zero_oor"] += int(z.sum())
            cnt["rerounded"] += int((oor & ~all_zero).sum())
        byte = np.where(is_nan, np.uint8(0x7F), byte)
        cnt["nan"] += int(is_nan.sum())
        cnt["blocks"] += int(b.size)
        nv[m] = np.repeat(byte, 2, axis=-1)
        glob[m] = np.float32(np.ldexp(1.0, G))
    return nv, glob, cnt
