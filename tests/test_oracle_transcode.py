"""Pins for the oracle's MXFP4 -> NVFP4 transcode (CPU only).

The pages fix: codes unchanged, every block's value preserved exactly (two
E4M3 scales per 32-block times a power-of-two global), and the audit counts
(blocks = values / 32, no all-zero, no re-rounded block on the real model).
"""
import os

import numpy as np

import oracle
from synth import random_mx_small

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _counts():
    d = {}
    with open(os.path.join(GOLD, "page_counts.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                d[k] = int(v)
    return d


def _check_exact(packed, mx):
    nv, glob, cnt = oracle.transcode_mx_to_nv(mx, packed)
    a = oracle.dequant_mx(packed, mx)
    b = oracle.dequant_nv(packed, nv, glob)
    assert np.array_equal(a, b)                      # value-exact, every element
    assert np.array_equal(np.signbit(a), np.signbit(b))
    return nv, glob, cnt


def test_transcode_value_exact_random():
    packed, mx = random_mx_small(10, 6, 32, 256)          # scales 2^-8..2^-2
    nv, glob, cnt = _check_exact(packed, mx)
    assert cnt == {"blocks": 6 * 32 * 8, "zero_oor": 0, "rerounded": 0, "nan": 0}
    # the two 16-halves of each 32-block carry the same byte
    assert np.array_equal(nv[..., 0::2], nv[..., 1::2])
    # the largest block scale maps to 2^8 = 256 (E4M3 0x78)
    for m in range(6):
        assert nv[m].max() == 0x78
        assert glob[m] == np.float32(2.0 ** (int(mx[m].max()) - 127 - 8))


def test_transcode_value_exact_span_17():
    # block exponents spanning 17 binades are still exact (2^8 .. 2^-9 in E4M3)
    packed, mx = random_mx_small(11, 3, 16, 128, lo=100, hi=117)
    assert mx.max() - mx.min() <= 17
    nv, glob, cnt = _check_exact(packed, mx)
    assert cnt["rerounded"] == 0 and cnt["zero_oor"] == 0


def test_transcode_decode_shape_bytes():
    # E8M0 scales 2^-8..2^-2: G = -10 and every E4M3 byte is a power of two 2^2..2^8
    packed, mx = random_mx_small(12, 4, 64, 512)
    nv, glob, cnt = _check_exact(packed, mx)
    assert np.all(glob == np.float32(2.0 ** -10))
    assert set(np.unique(nv)) <= {0x48, 0x50, 0x58, 0x60, 0x68, 0x70, 0x78}


def test_transcode_out_of_range_blocks():
    packed, mx = random_mx_small(13, 1, 4, 128, lo=120, hi=120)
    mx = mx.copy()
    packed = packed.copy()
    mx[0, 0, 0] = 138                 # e_max = 11 -> G = 3
    mx[0, 1, 0] = 120                 # k = -7 - 3 = -10: below 2^-9, codes non-zero -> re-rounded
    mx[0, 2, 0] = 121                 # k = -9: exact (span 17)
    mx[0, 3, 1] = 100                 # far below range, codes forced to +-0 -> all-zero block
    packed[0, 3, 16:32] = np.array([0x00, 0x88, 0x80, 0x08] * 4, np.uint8)
    mx[0, 3, 2] = 255                 # NaN scale
    nv, glob, cnt = oracle.transcode_mx_to_nv(mx, packed)
    assert glob[0] == np.float32(8.0)
    assert cnt["blocks"] == 16
    assert cnt["nan"] == 1 and nv[0, 3, 4] == 0x7F and nv[0, 3, 5] == 0x7F
    assert cnt["zero_oor"] == 1 and nv[0, 3, 2] == 0x00
    assert nv[0, 2, 0] == 0x01
    # k = -10 is clamped to 2^-9 and counted; all other blocks k = -10 too (120 vs e_max 138)
    e = mx[0].astype(np.int64) - 127
    assert cnt["rerounded"] == int(np.sum((e - 3 < -9) & (mx[0] != 255))) - 1 == 12
    assert nv[0, 1, 0] == 0x01


def test_transcode_block_count_matches_pages():
    c = _counts()
    assert c["expert_values"] % 32 == 0
    assert c["expert_values"] // 32 == c["expert_scale_blocks"]
    # 47 layers x 256 experts x 3 matrices of 4096 x 2048 values
    assert c["expert_matrices"] == c["moe_layers"] * c["routed_experts"] * 3
    assert c["layer_expert_pairs"] == c["moe_layers"] * c["routed_experts"]
    per_matrix = c["expert_values"] // c["expert_matrices"]
    assert per_matrix == 4096 * 2048
    # the oracle's block counter for one such matrix, scaled, gives the page's count
    packed = np.zeros((1, 4096, 1024), np.uint8)
    mx = np.full((1, 4096, 64), 120, np.uint8)
    _, _, cnt = oracle.transcode_mx_to_nv(mx, packed)
    assert cnt["blocks"] * c["expert_matrices"] == c["expert_scale_blocks"]
    assert c["all_zero_blocks"] == 0 and c["rerounded_blocks"] == 0


# ------------------------------------------------ compact storage (4.125 b/w)
def test_compact_is_4p125_bits_and_lossless_on_model_shaped_data():
    """The compact encoding of model-shaped MXFP4 weights takes 4.125 bits per
    weight (the page's figure) and gives back exactly the MXFP4 values."""
    from synth import WORKLOADS, expert_weights
    W = expert_weights(WORKLOADS["decode"], experts=[0, 1])
    for name in ("gate", "down"):
        packed, mx = W[name]
        c4, base, cnt = oracle.compact_mx(mx, packed)
        assert cnt["rerounded"] == 0 and cnt["nan"] == 0 and cnt["blocks"] == mx.size
        n_vals = packed.size * 2
        assert (packed.nbytes + c4.nbytes) * 8 / n_vals == 4.125
        for e in range(2):
            assert np.array_equal(oracle.dequant_compact(packed[e], c4[e], base[e]),
                                  oracle.dequant_mx(packed[e], mx[e]))


def test_compact_edge_blocks():
    """Span 15 below the largest exponent is exact; span 16 is re-rounded unless
    the block is all zero; NaN has no code."""
    from synth import random_mx_small
    packed, mx = random_mx_small(31, 3, 16, 256, lo=110, hi=125)   # span 15: every block exact
    packed = packed.copy()
    mx = mx.copy()
    c4, base, cnt = oracle.compact_mx(mx, packed)
    assert cnt["rerounded"] == 0 and cnt["zero_oor"] == 0
    for e in range(3):
        assert np.array_equal(oracle.dequant_compact(packed[e], c4[e], base[e]), oracle.dequant_mx(packed[e], mx[e]))
    mx[1, 2, 3] = 109                      # 16 below the largest: not expressible
    mx[1, 4, 0] = 100
    packed[1, 4, 0:16] = 0x88              # ... but all -0 codes: exact
    mx[2, 0, 1] = 255                      # NaN
    c4, base, cnt = oracle.compact_mx(mx, packed)
    assert cnt["rerounded"] == 1 and cnt["zero_oor"] == 1 and cnt["nan"] == 1
    assert np.array_equal(oracle.dequant_compact(packed[0], c4[0], base[0]), oracle.dequant_mx(packed[0], mx[0]))
    d = oracle.dequant_compact(packed[1], c4[1], base[1])
    assert np.all(d[4, 0:32] == 0)
