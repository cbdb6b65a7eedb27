"""Every output row of the MFMA-tiled ("prefill") grouped GEMM kernels against
the oracle, on shapes that give every persistent workgroup several tiles.

The persistent kernels walk a tile list (expert, n-tile, m-tile) cut into one
contiguous slice per XCD.  The bf16-token 64 x 512 kernel at these sizes
(~700 rows per expert) carries its load pipeline from each tile into the
next (the next tile's first steps load during the current tile's last ones);
the others restart it on each tile.  These shapes make 1,000-1,600 tiles for
256 workgroups (4-6 tiles each), with ragged experts (tails of every length,
empty experts) so that slice boundaries fall inside experts.  Each case is
checked on every row:
  * bf16 tokens, 64 x 512 tiles (SwiGLU gate/up and down), row-major and tiled;
  * bf16 tokens, 128 x 256 tiles (N a multiple of 256 but not 512);
  * NVFP4 tokens (codes + scales dequantised in the kernel), 128 x 256 tiles.
z and o are bf16-stored sums: within max(2e-2 rms, one bf16 ulp) of the oracle
element by element (the FP32 and float64 sums may round to neighbouring bf16
values).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_ULP, assert_close_rms, bf16_to_f64, dev_bf16, dev_f32, dev_i32, dev_u8, host, host_bf16_bits, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_group_amd as moe  # noqa: E402

E = 32


def _counts(seed, mean):
    """Ragged per-expert row counts around `mean`: two empty experts, tails of
    every length modulo the 64- and 128-row tiles."""
    rng = np.random.default_rng(seed)
    c = rng.integers(mean // 2, mean * 3 // 2, size=E)
    c[[5, 17]] = 0
    c[3] = 1
    c[9] = 63
    c[10] = 129
    return c.astype(np.int64)


def _weights(seed, n, k, tiled):
    packed, mx = synth.random_mx_small(seed, E, n, k)
    w = moe.Weights(dev_u8(packed), dev_u8(mx))
    if tiled:
        w = moe.tile_weights(w)
    dq = [oracle.dequant_mx(packed[e], mx[e]) for e in range(E)]
    return w, dq


def _tiles(counts, bm, ntn):
    return int(np.sum(-(-counts // bm)) * ntn)


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("amode", ["bf16", "nvfp4"])
def test_swiglu_every_row(tiled, amode):
    """gate/up + SwiGLU, H = 2048, I = 1024: 64 x 512 tiles (bf16 tokens) or
    128 x 256 (NVFP4 tokens), ~700 rows per expert."""
    H, I = 2048, 1024
    counts = _counts(1, 700)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    tiles = _tiles(counts, 64, I // 256) if amode == "bf16" else _tiles(counts, 128, I // 128)
    say(f"swiglu every row tiled={tiled} amode={amode} R={R} tiles={tiles}")
    assert tiles >= 4 * 256
    tsrc = 4096
    x = synth.random_bf16(201, (tsrc, H))
    gather = np.random.default_rng(202).integers(0, tsrc * 8, size=R).astype(np.int32)
    wg, dg = _weights(203, I, H, tiled)
    wu, du = _weights(204, I, H, tiled)
    if amode == "nvfp4":
        xc, xs = oracle.quantize_nvfp4(x, 1.0)
        a_val, a_dev, a_sc = oracle.dequant_nvfp4_act(xc, xs), dev_u8(xc), dev_u8(xs)
    else:
        a_val, a_dev, a_sc = bf16_to_f64(x), dev_bf16(x), None
    z = moe.grouped_gemm(a_dev, wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8, a_scales=a_sc,
                         algo=moe.MOE_ALGO_PREFILL)
    torch.cuda.synchronize()
    zb = bf16_to_f64(host_bf16_bits(z))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        a = a_val[gather[r0:r1] // 8]
        ref = bf16_to_f64(oracle.round_to_bf16_bits(oracle.silu(a @ dg[e].T) * (a @ du[e].T)))
        assert_close_rms(zb[r0:r1], ref, what=f"z expert {e} ({r1 - r0} rows)", ulp_rel=BF16_ULP)


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("amode", ["bf16", "nvfp4"])
def test_down_every_row(tiled, amode):
    """down projection, N = H = 2048, K = I = 1024: 64 x 512 tiles (bf16) or
    128 x 256 (NVFP4 tokens), ~700 rows per expert; the rows past
    expert_offsets[E] keep their previous contents."""
    H, I = 2048, 1024
    counts = _counts(2, 700)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    tiles = _tiles(counts, 64, H // 512) if amode == "bf16" else _tiles(counts, 128, H // 256)
    say(f"down every row tiled={tiled} amode={amode} R={R} tiles={tiles}")
    assert tiles >= 4 * 256
    zin = synth.random_bf16(211, (R + 7, I))
    wd, dd = _weights(212, H, I, tiled)
    if amode == "nvfp4":
        zc, zs = oracle.quantize_nvfp4(zin, 1.0)
        a_val, a_dev, a_sc = oracle.dequant_nvfp4_act(zc, zs), dev_u8(zc), dev_u8(zs)
    else:
        a_val, a_dev, a_sc = bf16_to_f64(zin), dev_bf16(zin), None
    out = torch.full((R + 7, H), 3.0, dtype=torch.bfloat16, device="cuda")
    moe.grouped_gemm(a_dev, wd, None, dev_i32(offsets), R + 7, a_scales=a_sc, out=out, algo=moe.MOE_ALGO_PREFILL)
    torch.cuda.synchronize()
    ob = host_bf16_bits(out)
    assert np.all(bf16_to_f64(ob[R:]) == 3.0), "rows past expert_offsets[E] were written"
    ov = bf16_to_f64(ob[:R])
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        assert_close_rms(ov[r0:r1], a_val[r0:r1] @ dd[e].T, what=f"o expert {e} ({r1 - r0} rows)", ulp_rel=BF16_ULP)


def test_tall_bf16_tiles_every_row():
    """bf16 tokens on 128 x 256 tiles: SwiGLU with I = 640 (a multiple of 128
    outputs per matrix, not of 256) and down with N = 1792 (a multiple of 256,
    not of 512), ~1100 rows per expert."""
    H, I, Hd, Id = 2048, 640, 1792, 1024
    counts = _counts(3, 1100)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    say(f"tall bf16 tiles R={R} tiles swiglu={_tiles(counts, 128, I // 128)} down={_tiles(counts, 128, Hd // 256)}")
    assert _tiles(counts, 128, I // 128) >= 4 * 256 and _tiles(counts, 128, Hd // 256) >= 4 * 256
    tsrc = 4096
    x = synth.random_bf16(221, (tsrc, H))
    gather = np.random.default_rng(222).integers(0, tsrc * 8, size=R).astype(np.int32)
    wg, dg = _weights(223, I, H, False)
    wu, du = _weights(224, I, H, False)
    wd, dd = _weights(225, Hd, Id, False)
    zin = synth.random_bf16(226, (R, Id))
    z = moe.grouped_gemm(dev_bf16(x), wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8,
                         algo=moe.MOE_ALGO_PREFILL)
    o = moe.grouped_gemm(dev_bf16(zin), wd, None, dev_i32(offsets), R, algo=moe.MOE_ALGO_PREFILL)
    torch.cuda.synchronize()
    zb, ob = bf16_to_f64(host_bf16_bits(z)), bf16_to_f64(host_bf16_bits(o))
    xv, zv = bf16_to_f64(x), bf16_to_f64(zin)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        a = xv[gather[r0:r1] // 8]
        zref = bf16_to_f64(oracle.round_to_bf16_bits(oracle.silu(a @ dg[e].T) * (a @ du[e].T)))
        assert_close_rms(zb[r0:r1], zref, what=f"z expert {e}", ulp_rel=BF16_ULP)
        assert_close_rms(ob[r0:r1], zv[r0:r1] @ dd[e].T, what=f"o expert {e}", ulp_rel=BF16_ULP)


def _pad_experts(w, extra):
    """The same weights with `extra` all-zero experts appended (never read: no rows)."""
    pad = lambda t: torch.cat([t, torch.zeros((extra,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)])
    return moe.Weights(pad(w.packed), pad(w.scale))


@pytest.mark.parametrize("swiglu", [True, False])
def test_cross_tile_kernel_equals_per_tile_kernel(swiglu):
    """bf16 tokens on 64 x 512 tiles run one of two kernels: with at least 160
    rows per expert on average the pipeline runs on across tiles, below that it
    restarts per tile (and skips the empty 16-row blocks of a tile).  Both add
    the same products in the same order, so the same call with 128 more empty
    experts (the average falls below 160 rows) gives the same bytes; the rows
    are also checked against the oracle."""
    H, I = 2048, 1024
    counts = _counts(4, 700)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    extra = 128
    assert R >= 160 * E and R < 160 * (E + extra)
    offsets2 = np.concatenate([offsets, np.full(extra, R)]).astype(np.int32)
    say(f"cross-tile vs per-tile swiglu={swiglu} R={R}")
    if swiglu:
        tsrc = 4096
        x = synth.random_bf16(231, (tsrc, H))
        gather = np.random.default_rng(232).integers(0, tsrc * 8, size=R).astype(np.int32)
        wg0, dg = _weights(233, I, H, False)
        wu0, du = _weights(234, I, H, False)
        wg, wu = moe.tile_weights(wg0), moe.tile_weights(wu0)
        wg2, wu2 = moe.tile_weights(_pad_experts(wg0, extra)), moe.tile_weights(_pad_experts(wu0, extra))
        args = dict(gather=dev_i32(gather), gather_div=8, algo=moe.MOE_ALGO_PREFILL)
        y1 = moe.grouped_gemm(dev_bf16(x), wg, wu, dev_i32(offsets), R, **args)
        y2 = moe.grouped_gemm(dev_bf16(x), wg2, wu2, dev_i32(offsets2), R, **args)
        a_all = bf16_to_f64(x)[gather // 8]
        ref = lambda e, r0, r1: bf16_to_f64(oracle.round_to_bf16_bits(
            oracle.silu(a_all[r0:r1] @ dg[e].T) * (a_all[r0:r1] @ du[e].T)))
    else:
        zin = synth.random_bf16(235, (R, I))
        wd0, dd = _weights(236, H, I, False)
        wd, wd2 = moe.tile_weights(wd0), moe.tile_weights(_pad_experts(wd0, extra))
        y1 = moe.grouped_gemm(dev_bf16(zin), wd, None, dev_i32(offsets), R, algo=moe.MOE_ALGO_PREFILL)
        y2 = moe.grouped_gemm(dev_bf16(zin), wd2, None, dev_i32(offsets2), R, algo=moe.MOE_ALGO_PREFILL)
        zv = bf16_to_f64(zin)
        ref = lambda e, r0, r1: zv[r0:r1] @ dd[e].T
    torch.cuda.synchronize()
    b1, b2 = host_bf16_bits(y1), host_bf16_bits(y2)
    assert np.array_equal(b1, b2), f"{int(np.sum(b1 != b2))} outputs differ between the two kernels"
    yv = bf16_to_f64(b1)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            assert_close_rms(yv[r0:r1], ref(e, r0, r1), what=f"expert {e} ({r1 - r0} rows)", ulp_rel=BF16_ULP)
