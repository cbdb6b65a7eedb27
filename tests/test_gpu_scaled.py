"""GPU parity of the block-scaled MFMA path: MXFP8 activations (W4A8) and NVFP4
activations as exact E4M3 planes (W4A4), both with the FP4 weights as the
native MFMA operand.

  * quantisers: MXFP8 codes and scales byte-exact against the oracle; the
    NVFP4 planes decoded here (E4M3 bytes x E8M0 scales) equal the oracle's
    NVFP4 values exactly;
  * grouped GEMMs on every row, on shapes with several tiles per persistent
    workgroup: z and o against the oracle from the same quantised operands
    (bf16-stored sums: within max(2e-2 rms, one bf16 ulp)), and the quantised
    z outputs exactly the oracle's quantisation of the GPU's own bf16 z.
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


def decode_planes(planes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3 planes [rows, 2k] + E8M0 [rows, k/16] -> float64 [rows, k]: per 16-value
    block, bytes 0..15 are the hi plane, 16..31 the lo plane, both times the block's scale."""
    rows, k2 = planes.shape
    p = planes.reshape(rows, k2 // 32, 2, 16)
    v = oracle.e4m3_value(p[:, :, 0, :]) + oracle.e4m3_value(p[:, :, 1, :])
    return (v * oracle.e8m0_value(scales)[..., None]).reshape(rows, k2 // 2)


def _wide_input(seed, rows, k):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, k)) * 10.0 ** rng.integers(-5, 5, (rows, 1))).astype(np.float32)
    x[0, :64] = 0.0
    x[0, 64:96] = -0.0
    x[1, :32] = 0.25
    x[1, 0] = 1.875 * 2 ** 3                      # saturates at 448 * X
    x[2, :32] = 2.0 ** -20
    x[2, 0] = 1.0                                 # E4M3 subnormals / flush to zero
    for j, amax in enumerate(synth.OUTLIER_AMAX):
        x[3 + j, 7] = -amax
    return synth.bf16_bits_from_f32(x)


def test_quantize_mxfp8_parity():
    xb = _wide_input(301, 203, 512)
    c_ref, s_ref = oracle.quantize_mxfp8(xb)
    c, s = moe.quantize_mxfp8(dev_bf16(xb))
    torch.cuda.synchronize()
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(c), c_ref)


@pytest.mark.parametrize("g", [1.0, 0.5, 4.0])
def test_quantize_planes_values(g):
    xb = _wide_input(302, 203, 512)
    p, ps = moe.quantize_nvfp4_planes(dev_bf16(xb), g)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.quantize_nvfp4(xb, g)
    want = oracle.dequant_nvfp4_act(c_ref, s_ref, g)
    got = decode_planes(host(p), host(ps))
    assert np.array_equal(got, want)


E = 32


def _counts(seed, mean):
    rng = np.random.default_rng(seed)
    c = rng.integers(mean // 2, mean * 3 // 2, size=E)
    c[[5, 17]] = 0
    c[3] = 1
    c[9] = 63
    c[10] = 129
    return c.astype(np.int64)


def _weights(seed, n, k, fmt, tiled):
    packed, mx = synth.random_mx_small(seed, E, n, k)
    if fmt == "mx":
        w = moe.Weights(dev_u8(packed), dev_u8(mx))
    else:
        sc, g, cnt = oracle.transcode_mx_to_nv(mx, packed)
        assert cnt["rerounded"] == 0
        w = moe.Weights(dev_u8(packed), dev_u8(sc), dev_f32(g), scales_pow2=True, mx_exact=True)
    if tiled:
        w = moe.tile_weights(w)
    return w, [oracle.dequant_mx(packed[e], mx[e]) for e in range(E)]


def _act(xb, mode):
    """(device operand, device scales, float64 values the oracle multiplies)."""
    if mode == "mxfp8":
        c, s = oracle.quantize_mxfp8(xb)
        return dev_u8(c), dev_u8(s), oracle.dequant_mxfp8(c, s)
    p, ps = moe.quantize_nvfp4_planes(dev_bf16(xb), 1.0)        # planes: values checked above
    c, s = oracle.quantize_nvfp4(xb, 1.0)
    return p, ps, oracle.dequant_nvfp4_act(c, s)


@pytest.mark.parametrize("mode", ["mxfp8", "planes"])
@pytest.mark.parametrize("fmt,tiled", [("mx", False), ("mx", True), ("nv", False), ("nv", True)])
def test_scaled_swiglu_every_row(mode, fmt, tiled):
    """gate/up + SwiGLU on the block-scaled MFMA, H = 2048, I = 1024, ~700 rows per
    expert (1,200+ tiles of 64 x 512 for 256 workgroups); z on every row, and the
    quantised z output exactly the oracle's quantisation of the GPU's bf16 z."""
    H, I = 2048, 1024
    counts = _counts(11, 700)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    say(f"scaled swiglu mode={mode} fmt={fmt} tiled={tiled} R={R}")
    tsrc = 4096
    xb = synth.random_bf16(311, (tsrc, H))
    gather = np.random.default_rng(312).integers(0, tsrc * 8, size=R).astype(np.int32)
    wg, dg = _weights(313, I, H, fmt, tiled)
    wu, du = _weights(314, I, H, fmt, tiled)
    a_dev, a_sc, a_val = _act(xb, mode)
    if mode == "mxfp8":
        zq = torch.empty((R, I), dtype=torch.uint8, device="cuda")
        zs = torch.empty((R, I // 32), dtype=torch.uint8, device="cuda")
    else:
        zq = torch.empty((R, 2 * I), dtype=torch.uint8, device="cuda")
        zs = torch.empty((R, I // 16), dtype=torch.uint8, device="cuda")
    z = moe.grouped_gemm(a_dev, wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8, a_scales=a_sc,
                         out_codes=zq, out_scales=zs, a_mode=mode, out_format=mode)
    torch.cuda.synchronize()
    zb = host_bf16_bits(z)
    zv = bf16_to_f64(zb)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        a = a_val[gather[r0:r1] // 8]
        ref = bf16_to_f64(oracle.round_to_bf16_bits(oracle.silu(a @ dg[e].T) * (a @ du[e].T)))
        assert_close_rms(zv[r0:r1], ref, what=f"z expert {e} ({r1 - r0} rows)", ulp_rel=BF16_ULP)
    if mode == "mxfp8":
        c_ref, s_ref = oracle.quantize_mxfp8(zb)
        assert np.array_equal(host(zs), s_ref)
        assert np.array_equal(host(zq), c_ref)
    else:
        c_ref, s_ref = oracle.quantize_nvfp4(zb, 1.0)
        assert np.array_equal(decode_planes(host(zq), host(zs)), oracle.dequant_nvfp4_act(c_ref, s_ref))


@pytest.mark.parametrize("mode", ["mxfp8", "planes"])
@pytest.mark.parametrize("fmt,tiled", [("mx", False), ("nv", True)])
def test_scaled_down_every_row(mode, fmt, tiled):
    """down projection on the block-scaled MFMA, N = 2048, K = 1024: o on every row;
    rows past expert_offsets[E] keep their contents."""
    H, I = 2048, 1024
    counts = _counts(12, 700)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    say(f"scaled down mode={mode} fmt={fmt} tiled={tiled} R={R}")
    zin = synth.random_bf16(321, (R + 7, I), std=3.0)
    wd, dd = _weights(322, H, I, fmt, tiled)
    a_dev, a_sc, a_val = _act(zin, mode)
    out = torch.full((R + 7, H), 3.0, dtype=torch.bfloat16, device="cuda")
    moe.grouped_gemm(a_dev, wd, None, dev_i32(offsets), R + 7, a_scales=a_sc, out=out, a_mode=mode)
    torch.cuda.synchronize()
    ob = host_bf16_bits(out)
    assert np.all(bf16_to_f64(ob[R:]) == 3.0), "rows past expert_offsets[E] were written"
    ov = bf16_to_f64(ob[:R])
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        assert_close_rms(ov[r0:r1], a_val[r0:r1] @ dd[e].T, what=f"o expert {e}", ulp_rel=BF16_ULP)


@pytest.mark.parametrize("mode", ["mxfp8", "planes"])
def test_scaled_small_batches(mode):
    """Few rows per expert (decode-sized, every tile mostly padding) at the model's K."""
    H, I = 4096, 2048
    Es = 8
    counts = np.array([1, 0, 3, 8, 0, 2, 17, 5])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    xb = synth.random_bf16(331, (8, H))
    gather = np.random.default_rng(332).integers(0, 64, size=R).astype(np.int32)
    packed, mx = synth.random_mx_small(333, Es, I, H)
    pu, mu = synth.random_mx_small(334, Es, I, H)
    wg, wu = moe.Weights(dev_u8(packed), dev_u8(mx)), moe.Weights(dev_u8(pu), dev_u8(mu))
    a_dev, a_sc, a_val = _act(xb, mode)
    z = moe.grouped_gemm(a_dev, wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8, a_scales=a_sc,
                         a_mode=mode)
    torch.cuda.synchronize()
    zv = bf16_to_f64(host_bf16_bits(z))
    for e in range(Es):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        a = a_val[gather[r0:r1] // 8]
        g = a @ oracle.dequant_mx(packed[e], mx[e]).T
        u = a @ oracle.dequant_mx(pu[e], mu[e]).T
        ref = bf16_to_f64(oracle.round_to_bf16_bits(oracle.silu(g) * u))
        assert_close_rms(zv[r0:r1], ref, what=f"z expert {e}", ulp_rel=BF16_ULP)


def test_scaled_rejects_unsupported():
    """Shapes and weights the block-scaled kernels do not cover are refused, not run."""
    w = moe.Weights(dev_u8(np.zeros((2, 384, 1024), np.uint8)), dev_u8(np.full((2, 384, 64), 127, np.uint8)))
    a = torch.zeros((4, 2048), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    off = dev_i32(np.array([0, 2, 4], np.int32))
    with pytest.raises(moe.MoeError) as ei:           # n = 384 is not a multiple of 512
        moe.grouped_gemm(a, w, None, off, 4, a_scales=s, a_mode="mxfp8")
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    nv = moe.Weights(dev_u8(np.zeros((2, 512, 1024), np.uint8)), dev_u8(np.zeros((2, 512, 128), np.uint8)),
                     dev_f32(np.ones(2, np.float32)), scales_pow2=True)
    with pytest.raises(moe.MoeError) as ei:           # NV weights without the exact-transcode flag
        moe.grouped_gemm(a, nv, None, off, 4, a_scales=s, a_mode="mxfp8")
    assert ei.value.status == moe.MOE_ERR_INVALID
