"""GPU parity of each kernel against the CPU oracle, through the C ABI.

Exact comparisons for integer / byte results (routing ids, permutation,
transcoded scales and counters, NVFP4 codes); max|err| <= 2e-2 * rms for
floating-point outputs; router weights to rtol 1e-6.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (BF16_ULP, assert_close_rms, bf16_to_f64, dev_bf16, dev_f32, dev_i32, dev_u8, host, host_bf16_bits,
                      say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_group_amd as moe  # noqa: E402


def test_native_library_is_loaded():
    maps = open("/proc/self/maps").read()
    assert "libmoefp4.so" in maps
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    say("  HIP runtime(s):", hip)
    assert len(hip) == 1, f"more than one HIP runtime mapped: {hip}"
    assert moe.lib.moe_version().decode().startswith("moe_fp4")


# ------------------------------------------------------------------ route
ROUTE_CASES = [
    ("tiny", 32, False), ("decode", 1, False), ("decode", 64, False), ("prefill", 8192, True),
    ("reap50", 16384, False),
]


@pytest.mark.parametrize("name,T,with_bias", ROUTE_CASES)
def test_route_parity(name, T, with_bias):
    w = synth.WORKLOADS[name]
    s = w.shape
    say(f"route {name} T={T}")
    l = synth.logits(w, T)
    bias = synth.correction_bias(w) if with_bias else None
    r = oracle.route(l, bias, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
    ids, wts = moe.route(dev_f32(l), None if bias is None else dev_f32(bias), s.num_experts, s.n_group,
                         s.topk_group, s.top_k, s.routed_scaling_factor)
    torch.cuda.synchronize()
    gi, gw = host(ids), host(wts)
    say(f"  near-ties flagged: {int(r.near_tie.sum())}")
    assert not r.near_tie.any(), "a routing decision of this workload lies within 1e-12 of a tie"
    assert np.array_equal(gi, r.ids)
    np.testing.assert_allclose(gw, r.weights, rtol=1e-6)


def test_route_ties_and_edge_cases():
    # all-equal scores, duplicated logits across groups, a strong bias, tiny T
    E = 256
    l = np.zeros((6, E), np.float32)
    l[1] = synth.random_logits(1, 1, E)[0]
    l[1, 100] = l[1, 7]                      # exact duplicate in another group
    l[2, :] = 3.0
    l[2, ::17] = 5.0
    l[3] = synth.random_logits(2, 1, E)[0] * 8          # saturating sigmoids
    l[4] = -l[3]
    l[5] = synth.random_logits(3, 1, E)[0]
    bias = np.zeros(E, np.float32)
    bias[[5, 99, 200]] = [0.3, -0.2, 0.7]
    for b in (None, bias):
        r = oracle.route(l, b, 8, 4, 8, 2.827)
        ids, wts = moe.route(dev_f32(l), None if b is None else dev_f32(b), E, 8, 4, 8, 2.827)
        torch.cuda.synchronize()
        assert np.array_equal(host(ids), r.ids)
        np.testing.assert_allclose(host(wts), r.weights, rtol=1e-6)


@pytest.mark.parametrize("E,n_group,topk_group,top_k", [(64, 4, 2, 6), (128, 8, 4, 8), (16, 2, 1, 3)])
def test_route_other_shapes(E, n_group, topk_group, top_k):
    l = synth.random_logits(E, 257, E)
    r = oracle.route(l, None, n_group, topk_group, top_k, 1.5)
    ids, wts = moe.route(dev_f32(l), None, E, n_group, topk_group, top_k, 1.5)
    torch.cuda.synchronize()
    assert np.array_equal(host(ids), r.ids)
    np.testing.assert_allclose(host(wts), r.weights, rtol=1e-6)


# ---------------------------------------------------------------- permute
@pytest.mark.parametrize("T,E,invalid", [(0, 32, False), (1, 256, False), (7, 32, False), (64, 256, False),
                                          (255, 256, False), (300, 128, True), (4096, 256, False),
                                          (16384, 128, False), (2000, 1024, True)])
def test_permute_parity(T, E, invalid):
    rng = np.random.default_rng(T * 7 + E)
    ids = rng.integers(0, E, size=(T, 8)).astype(np.int32)
    if T > 100:     # skew: a few experts take many slots
        hot = rng.random((T, 8)) < 0.3
        ids[hot] = rng.integers(0, 3, size=int(hot.sum()))
    if invalid and T:
        ids[0, 0] = -1
        ids[T // 2, 3] = E
    say(f"permute T={T} E={E}")
    valid = (ids >= 0) & (ids < E)
    off_ref, ss_ref, sr_ref = oracle.permute(np.where(valid, ids, 0), E)
    off, ss, sr = moe.permute(dev_i32(ids), E)
    torch.cuda.synchronize()
    if invalid and T:
        # reference with the invalid slots removed
        flat = ids.ravel()
        keep = np.flatnonzero(valid.ravel())
        order = keep[np.argsort(flat[keep], kind="stable")]
        counts = np.bincount(flat[keep], minlength=E)
        off_ref = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        ss_ref = order.astype(np.int32)
        sr_ref = np.full(flat.size, -1, np.int32)
        sr_ref[order] = np.arange(order.size)
        n = order.size
        assert np.array_equal(host(off), off_ref)
        assert np.array_equal(host(ss)[:n], ss_ref)
        assert np.array_equal(host(sr), sr_ref)
        return
    assert np.array_equal(host(off), off_ref)
    assert np.array_equal(host(ss), ss_ref)
    assert np.array_equal(host(sr), sr_ref)


# --------------------------------------------------------- route + permute
@pytest.mark.parametrize("T,E,n_group,topk_group,top_k,with_bias", [
    (0, 256, 8, 4, 8, False), (1, 256, 8, 4, 8, False), (2, 256, 8, 4, 8, True), (3, 64, 4, 2, 6, False),
    (4, 256, 8, 4, 16, True), (4, 16, 2, 1, 3, False), (7, 256, 8, 4, 8, True), (8, 256, 8, 4, 8, False),
    (12, 64, 4, 2, 6, True), (16, 256, 8, 4, 16, True), (17, 256, 8, 4, 8, False), (64, 256, 8, 4, 8, True),
    (255, 256, 8, 4, 8, False), (256, 256, 8, 4, 8, False), (300, 256, 8, 4, 8, True), (513, 64, 4, 2, 6, False),
    (64, 16, 2, 1, 3, False)])
def test_route_permute_parity(T, E, n_group, topk_group, top_k, with_bias):
    """The fused call equals moe_route then moe_permute bit for bit (one launch
    up to 2048 slots, two launches above), the oracle on its ids, and leaves the
    hand-off counter at zero across calls."""
    rng = np.random.default_rng(T * 31 + E)
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    for rep in range(3):
        say(f"route_permute T={T} E={E} top_k={top_k} rep={rep}")
        l = synth.random_logits(T * 7 + rep, T, E) if T else np.zeros((0, E), np.float32)
        bias = (rng.standard_normal(E) * 0.1).astype(np.float32) if with_bias else None
        db = None if bias is None else dev_f32(bias)
        ids, wts, off, ss, sr = moe.route_permute(dev_f32(l), db, E, n_group, topk_group, top_k, 2.827, counter)
        ids2, wts2 = moe.route(dev_f32(l), db, E, n_group, topk_group, top_k, 2.827)
        off2, ss2, sr2 = moe.permute(ids2, E)
        torch.cuda.synchronize()
        assert int(host(counter)[0]) == 0
        for a, b in ((ids, ids2), (wts, wts2), (off, off2), (ss, ss2), (sr, sr2)):
            assert np.array_equal(host(a).view(np.int32), host(b).view(np.int32))
        if T:
            r = oracle.route(l, bias, n_group, topk_group, top_k, 2.827)
            assert not r.near_tie.any()
            assert np.array_equal(host(ids), r.ids)
            off_ref, ss_ref, sr_ref = oracle.permute(host(ids), E)
            assert np.array_equal(host(off), off_ref)
            assert np.array_equal(host(ss), ss_ref)
            assert np.array_equal(host(sr), sr_ref)
        else:
            assert np.array_equal(host(off), np.zeros(E + 1, np.int32))


# --------------------------------------------------------------- quantise
@pytest.mark.parametrize("g", [1.0, 0.5, 4.0])
def test_quantize_nvfp4_parity(g):
    rng = np.random.default_rng(11)
    rows, k = 203, 512
    x = (rng.standard_normal((rows, k)) * 10.0 ** rng.integers(-4, 4, (rows, 1))).astype(np.float32)
    x[0, :16] = np.array([6, 5, 4, 3.5, 3, 2.5, 2, 1.75, 1.5, 1.25, 1, .75, .5, .25, 0, -0.0]) * 3.0
    x[1, :32] = 0.0
    x[1, 32:48] = 1e-5
    x[2, 16:32] = -0.0
    for j, amax in enumerate(synth.OUTLIER_AMAX + (2688.0,)):
        x[3 + j, 5] = amax
        x[3 + j, 40] = -amax
    xb = synth.bf16_bits_from_f32(x)
    c_ref, s_ref = oracle.quantize_nvfp4(xb, g)
    dq = torch.empty((rows, k), dtype=torch.bfloat16, device="cuda")
    c, s = moe.quantize_nvfp4(dev_bf16(xb), g, dequant=dq)
    torch.cuda.synchronize()
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(c), c_ref)
    # the dequantised output holds exactly the NVFP4 values codes x scale x g
    assert np.array_equal(bf16_to_f64(host_bf16_bits(dq)), oracle.dequant_nvfp4_act(c_ref, s_ref, g))


def test_quantize_nvfp4_outlier_rows():
    z = synth.down_inputs_with_outliers(256, 2048, 311296.0)
    c_ref, s_ref = oracle.quantize_nvfp4(z, 1.0)
    c, s = moe.quantize_nvfp4(dev_bf16(z), 1.0)
    torch.cuda.synchronize()
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(c), c_ref)
    v = oracle.dequant_nvfp4_act(host(c), host(s))
    assert np.max(np.abs(v)) == 2688.0


# -------------------------------------------------------------- transcode
def _transcode_case(mx, packed):
    nv_ref, g_ref, cnt_ref = oracle.transcode_mx_to_nv(mx, packed)
    nv, g, cnt = moe.transcode_mx_to_nv(dev_u8(mx), dev_u8(packed))
    torch.cuda.synchronize()
    assert np.array_equal(host(nv), nv_ref)
    assert np.array_equal(host(g).view(np.uint32), g_ref.view(np.uint32))
    c = host(cnt)
    assert list(c) == [cnt_ref["blocks"], cnt_ref["zero_oor"], cnt_ref["rerounded"], cnt_ref["nan"]]
    return c


def test_transcode_parity_random():
    packed, mx = synth.random_mx_small(21, 12, 64, 512)
    c = _transcode_case(mx, packed)
    assert c[2] == 0 and c[1] == 0


def test_transcode_parity_edge_blocks():
    packed, mx = synth.random_mx_small(22, 5, 32, 256, lo=90, hi=140)
    mx = mx.copy()
    packed = packed.copy()
    mx[0, 0, 0] = 200                  # large span: many blocks out of range
    mx[1, 3, 2] = 255                  # NaN
    mx[2, 5, 1] = 0                    # 2^-127
    packed[2, 5, 16:32] = 0x80         # all -0 codes -> all-zero block
    mx[3] = 255                        # a matrix with no finite block
    mx[4, :, :] = 127
    mx[4, 0, 0] = 127 + 17             # span 17 exactly
    mx[4, 1, 0] = 127 - 1              # span 18 -> re-rounded
    c = _transcode_case(mx, packed)
    assert c[1] >= 1 and c[2] >= 1 and c[3] >= 32 * 8


def test_transcode_parity_full_matrix_shape():
    # a few matrices at the real [2048, 4096] and [4096, 2048] shapes
    w = synth.WORKLOADS["decode"]
    W = synth.expert_weights(w, experts=[0, 1, 2])
    for name in ("gate", "down"):
        packed, mx = W[name]
        c = _transcode_case(mx, packed)
        assert c[1] == 0 and c[2] == 0


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("with_resid", [False, True])
def test_combine_parity(with_resid):
    rng = np.random.default_rng(5)
    T, k, h = 37, 8, 512
    R = T * k
    o = synth.random_bf16(31, (R, h))
    perm = rng.permutation(R).astype(np.int32)
    perm[3] = -1
    wts = rng.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    resid = synth.random_bf16(32, (T, h)) if with_resid else None
    y = moe.combine(dev_bf16(o), dev_i32(perm), dev_f32(wts), None if resid is None else dev_bf16(resid))
    torch.cuda.synchronize()
    ov = bf16_to_f64(o)
    gathered = np.where(perm[:, None] >= 0, ov[np.maximum(perm, 0)], 0.0).reshape(T, k, h)
    ref = oracle.combine(gathered, wts.astype(np.float64), resid)
    got = bf16_to_f64(host_bf16_bits(y))
    assert_close_rms(got, bf16_to_f64(ref), what="combine y", ulp_rel=BF16_ULP)
    # one bf16 rounding of an FP32 sum: at most one bf16 ulp from the float64 result
    refv = bf16_to_f64(ref)
    assert np.all(np.abs(got - refv) <= np.abs(refv) * 2 ** -7 + 1e-30)


# ------------------------------------------------------------ grouped GEMM
def _gemm_problem(seed, E, n, k, counts, nsrc, fmt, general_nv=False, pow2_flag=True):
    """fmt "mx" or "nv"; NV scales are the exact transcode (powers of two; declared
    as such when pow2_flag) or, with general_nv, arbitrary E4M3 bytes."""
    rng = np.random.default_rng(seed)
    packed, mx = synth.random_mx_small(seed, E, n, k)
    if fmt == "mx":
        wt = (packed, mx)
        dq = [oracle.dequant_mx(packed[e], mx[e]) for e in range(E)]
        wdev = moe.Weights(dev_u8(packed), dev_u8(mx))
    else:
        if general_nv:
            sc = rng.integers(0x20, 0x60, size=(E, n, k // 16)).astype(np.uint8)   # arbitrary E4M3 scales
            g = rng.uniform(0.3, 3.0, E).astype(np.float32)
        else:
            sc, g, _ = oracle.transcode_mx_to_nv(mx, packed)
        wt = (packed, sc, g)
        dq = [oracle.dequant_nv(packed[e], sc[e], g[e]) for e in range(E)]
        wdev = moe.Weights(dev_u8(packed), dev_u8(sc), dev_f32(g), scales_pow2=(not general_nv) and pow2_flag)
    return wdev, dq


GEMM_COUNTS = [0, 1, 17, 300, 1000, 33, 0, 64]


@pytest.mark.parametrize("algo", [moe.MOE_ALGO_DECODE, moe.MOE_ALGO_PREFILL])
@pytest.mark.parametrize("fmt,general,flag", [("mx", False, True), ("nv", False, True), ("nv", False, False),
                                               ("nv", True, False)])
@pytest.mark.parametrize("amode", ["bf16", "nvfp4"])
def test_grouped_gemm_swiglu_parity(algo, fmt, general, flag, amode):
    E, H, I = 8, 512, 256
    counts = np.array(GEMM_COUNTS)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    tsrc = 700
    say(f"gemm swiglu algo={algo} fmt={fmt} general={general} pow2 flag={flag} amode={amode} R={R}")
    x = synth.random_bf16(41, (tsrc, H))
    rng = np.random.default_rng(42)
    gather = rng.integers(0, tsrc * 8, size=R).astype(np.int32)          # slot ids; row = slot // 8
    wg, dg = _gemm_problem(43, E, I, H, counts, tsrc, fmt, general, flag)
    wu, du = _gemm_problem(44, E, I, H, counts, tsrc, fmt, general, flag)
    if amode == "nvfp4":
        xc, xs = oracle.quantize_nvfp4(x, 1.0)
        a_val = oracle.dequant_nvfp4_act(xc, xs)
        a_dev, a_sc = dev_u8(xc), dev_u8(xs)
    else:
        a_val = bf16_to_f64(x)
        a_dev, a_sc = dev_bf16(x), None
    zc = torch.empty((R, I // 2), dtype=torch.uint8, device="cuda")
    zs = torch.empty((R, I // 16), dtype=torch.uint8, device="cuda")
    zdq = torch.empty((R, I), dtype=torch.bfloat16, device="cuda")
    z = moe.grouped_gemm(a_dev, wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8, a_scales=a_sc,
                         out_codes=zc, out_scales=zs, out_dequant=zdq, algo=algo)
    z2 = moe.grouped_gemm(a_dev, wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8, a_scales=a_sc,
                          algo=algo)
    torch.cuda.synchronize()
    zb = host_bf16_bits(z)
    assert np.array_equal(zb, host_bf16_bits(z2)), "not deterministic"
    ref = np.zeros((R, I))
    for e in range(E):
        rows = slice(offsets[e], offsets[e + 1])
        a = a_val[gather[rows] // 8]
        gt, up = a @ dg[e].T, a @ du[e].T
        ref[rows] = oracle.silu(gt) * up
    ref = bf16_to_f64(oracle.round_to_bf16_bits(ref))          # z is stored as bfloat16
    assert_close_rms(bf16_to_f64(zb), ref, what="z", ulp_rel=BF16_ULP)
    # NVFP4 output: exactly the oracle's quantisation of the GPU's own bf16 z
    c_ref, s_ref = oracle.quantize_nvfp4(zb, 1.0)
    assert np.array_equal(host(zs), s_ref)
    assert np.array_equal(host(zc), c_ref)
    # and the dequantised NVFP4 output holds exactly those values
    assert np.array_equal(bf16_to_f64(host_bf16_bits(zdq)), oracle.dequant_nvfp4_act(c_ref, s_ref))


@pytest.mark.parametrize("algo", [moe.MOE_ALGO_DECODE, moe.MOE_ALGO_PREFILL])
@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("amode", ["bf16", "nvfp4"])
def test_grouped_gemm_down_parity(algo, fmt, amode):
    E, H, I = 8, 512, 256
    counts = np.array(GEMM_COUNTS[::-1])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    say(f"gemm down algo={algo} fmt={fmt} amode={amode} R={R}")
    z = synth.random_bf16(51, (R + 5, I))
    wd, dd = _gemm_problem(52, E, H, I, counts, R, fmt)
    if amode == "nvfp4":
        zc, zs = oracle.quantize_nvfp4(z, 1.0)
        a_val = oracle.dequant_nvfp4_act(zc, zs)
        a_dev, a_sc = dev_u8(zc), dev_u8(zs)
    else:
        a_val = bf16_to_f64(z)
        a_dev, a_sc = dev_bf16(z), None
    # rows R .. R+4 are past expert_offsets[E]: the call must leave them as they were
    sentinel = torch.full((R + 5, H), -777.0, dtype=torch.bfloat16, device="cuda")
    o = moe.grouped_gemm(a_dev, wd, None, dev_i32(offsets), R + 5, a_scales=a_sc, out=sentinel.clone(), algo=algo)
    torch.cuda.synchronize()
    ob = host_bf16_bits(o)
    assert np.array_equal(ob[R:], host_bf16_bits(sentinel)[R:]), "rows past expert_offsets[E] were written"
    got = bf16_to_f64(ob[:R])
    ref = np.zeros((R, H))
    for e in range(E):
        rows = slice(offsets[e], offsets[e + 1])
        ref[rows] = a_val[rows] @ dd[e].T
    assert_close_rms(got, ref, what="o", ulp_rel=BF16_ULP)


def test_grouped_gemm_empty_and_invalid():
    E, H, I = 4, 256, 128
    wg, _ = _gemm_problem(61, E, I, H, None, 1, "mx")
    offsets = dev_i32(np.zeros(E + 1, np.int32))
    x = dev_bf16(synth.random_bf16(62, (4, H)))
    out = torch.full((4, I), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.grouped_gemm(x, wg, wg, offsets, 4, out=out)             # every expert empty: nothing written
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    with pytest.raises(moe.MoeError) as ei:
        moe.grouped_gemm(x, wg, wg, offsets, 4, out=out, input_scale=3.0,
                         a_scales=torch.zeros((4, H // 16), dtype=torch.uint8, device="cuda"))
    assert ei.value.status == moe.MOE_ERR_INVALID


@pytest.mark.parametrize("algo", [moe.MOE_ALGO_DECODE, moe.MOE_ALGO_PREFILL])
@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("amode", ["bf16", "nvfp4"])
def test_grouped_gemm_model_k(algo, fmt, amode):
    """The model's K (4096 for gate/up, 2048 for down) with ragged expert loads."""
    E, H, I = 4, 4096, 256
    counts = np.array([3, 0, 21, 40])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    say(f"gemm model-K algo={algo} fmt={fmt} amode={amode} R={R}")
    x = synth.random_bf16(71, (40, H))
    gather = np.random.default_rng(72).integers(0, 40 * 8, size=R).astype(np.int32)
    wg, dg = _gemm_problem(73, E, I, H, counts, 40, fmt)
    wu, du = _gemm_problem(74, E, I, H, counts, 40, fmt)
    wd, dd = _gemm_problem(75, E, 512, 2048, counts, R, fmt)
    if amode == "nvfp4":
        xc, xs = oracle.quantize_nvfp4(x, 1.0)
        a_val, a_dev, a_sc = oracle.dequant_nvfp4_act(xc, xs), dev_u8(xc), dev_u8(xs)
    else:
        a_val, a_dev, a_sc = bf16_to_f64(x), dev_bf16(x), None
    z = moe.grouped_gemm(a_dev, wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8, a_scales=a_sc,
                         algo=algo)
    z2 = synth.random_bf16(76, (R, 2048))
    if amode == "nvfp4":
        zc, zs = oracle.quantize_nvfp4(z2, 1.0)
        z_val, z_dev, z_sc = oracle.dequant_nvfp4_act(zc, zs), dev_u8(zc), dev_u8(zs)
    else:
        z_val, z_dev, z_sc = bf16_to_f64(z2), dev_bf16(z2), None
    o = moe.grouped_gemm(z_dev, wd, None, dev_i32(offsets), R, a_scales=z_sc, algo=algo)
    torch.cuda.synchronize()
    zref = np.zeros((R, I))
    oref = np.zeros((R, 512))
    for e in range(E):
        rows = slice(offsets[e], offsets[e + 1])
        a = a_val[gather[rows] // 8]
        zref[rows] = oracle.silu(a @ dg[e].T) * (a @ du[e].T)
        oref[rows] = z_val[rows] @ dd[e].T
    zref = bf16_to_f64(oracle.round_to_bf16_bits(zref))
    assert_close_rms(bf16_to_f64(host_bf16_bits(z)), zref, what="z", ulp_rel=BF16_ULP)
    assert_close_rms(bf16_to_f64(host_bf16_bits(o)), oref, what="o", ulp_rel=BF16_ULP)


PASS_COUNTS = [0, 1, 17, 150, 400, 33, 0, 64]      # 8-row passes: 0+1+3+19+50+5+0+8 per expert


@pytest.mark.parametrize("fmt,general,amode", [("mx", False, "bf16"), ("nv", False, "bf16"), ("nv", True, "nvfp4"),
                                               ("mx", False, "nvfp4")])
def test_grouped_gemm_many_passes_parity(fmt, general, amode):
    """The weight-streaming kernel at the model's K, forced on a ragged batch whose
    experts need many 8-row passes over the same weights (up to 50)."""
    E, H, I, D = 8, 4096, 1024, 256
    counts = np.array(PASS_COUNTS)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    tsrc = 300
    say(f"gemm many passes fmt={fmt} general={general} amode={amode} R={R}")
    x = synth.random_bf16(81, (tsrc, H))
    gather = np.random.default_rng(82).integers(0, tsrc * 8, size=R).astype(np.int32)
    wg, dg = _gemm_problem(83, E, I, H, counts, tsrc, fmt, general)
    wu, du = _gemm_problem(84, E, I, H, counts, tsrc, fmt, general)
    wd, dd = _gemm_problem(85, E, D, 2048, counts, R, fmt, general)
    if amode == "nvfp4":
        xc, xs = oracle.quantize_nvfp4(x, 1.0)
        a_val, a_dev, a_sc = oracle.dequant_nvfp4_act(xc, xs), dev_u8(xc), dev_u8(xs)
    else:
        a_val, a_dev, a_sc = bf16_to_f64(x), dev_bf16(x), None
    algo = moe.MOE_ALGO_DECODE
    zc = torch.empty((R, I // 2), dtype=torch.uint8, device="cuda")
    zs = torch.empty((R, I // 16), dtype=torch.uint8, device="cuda")
    z = moe.grouped_gemm(a_dev, wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8, a_scales=a_sc,
                         out_codes=zc, out_scales=zs, algo=algo)
    z_again = moe.grouped_gemm(a_dev, wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8,
                               a_scales=a_sc, algo=algo)
    z2 = synth.random_bf16(86, (R, 2048))
    o = moe.grouped_gemm(dev_bf16(z2), wd, None, dev_i32(offsets), R, algo=algo)
    torch.cuda.synchronize()
    zb = host_bf16_bits(z)
    assert np.array_equal(zb, host_bf16_bits(z_again)), "not deterministic"
    zref = np.zeros((R, I))
    oref = np.zeros((R, D))
    z2v = bf16_to_f64(z2)
    for e in range(E):
        rows = slice(offsets[e], offsets[e + 1])
        a = a_val[gather[rows] // 8]
        zref[rows] = oracle.silu(a @ dg[e].T) * (a @ du[e].T)
        oref[rows] = z2v[rows] @ dd[e].T
    zref = bf16_to_f64(oracle.round_to_bf16_bits(zref))
    assert_close_rms(bf16_to_f64(zb), zref, what="z", ulp_rel=BF16_ULP)
    assert_close_rms(bf16_to_f64(host_bf16_bits(o)), oref, what="o", ulp_rel=BF16_ULP)
    c_ref, s_ref = oracle.quantize_nvfp4(zb, 1.0)
    assert np.array_equal(host(zs), s_ref)
    assert np.array_equal(host(zc), c_ref)


def _tile_ref(codes, scales, nv):
    """The tiled layout as the C header defines it, by reshaping (numpy)."""
    E, n, kb = codes.shape
    k = 2 * kb
    c = codes.reshape(E, n // 16, 16, k // 128, 4, 16)              # e, t, r, s, c, b
    c = c.transpose(0, 1, 3, 4, 2, 5).reshape(E, n, kb)             # e, t, s, c, r, b
    G = 32 if nv else 16
    sc = scales.reshape(E, n // 16, 16, k // 512, G)                # e, t, r, w, g
    sc = sc.transpose(0, 1, 3, 2, 4).reshape(scales.shape)          # e, t, w, r, g
    return np.ascontiguousarray(c), np.ascontiguousarray(sc)


@pytest.mark.parametrize("nv", [False, True])
def test_tile_weights_layout(nv):
    E, n, k = 3, 48, 1536
    say(f"tile weights nv={nv} E={E} n={n} k={k}")
    rng = np.random.default_rng(91)
    codes = rng.integers(0, 256, size=(E, n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(E, n, k // (16 if nv else 32)), dtype=np.uint8)
    g = dev_f32(np.ones(E, np.float32)) if nv else None
    w = moe.tile_weights(moe.Weights(dev_u8(codes), dev_u8(scales), g))
    torch.cuda.synchronize()
    c_ref, s_ref = _tile_ref(codes, scales, nv)
    assert w.tiled
    assert np.array_equal(host(w.packed), c_ref)
    assert np.array_equal(host(w.scale), s_ref)


@pytest.mark.parametrize("algo", [moe.MOE_ALGO_DECODE, moe.MOE_ALGO_PREFILL])
@pytest.mark.parametrize("fmt,general,amode", [("mx", False, "bf16"), ("nv", False, "bf16"), ("nv", True, "nvfp4"),
                                               ("mx", False, "nvfp4")])
def test_grouped_gemm_tiled_is_bitwise_row_major(algo, fmt, general, amode):
    """Same values in another order: the tiled layout gives bit-identical outputs
    (SwiGLU at K 4096 and down at K 2048, ragged experts with many 8-row passes)."""
    E, H, I, D = 8, 4096, 512, 256
    counts = np.array(PASS_COUNTS)
    offsets = dev_i32(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    R = int(counts.sum())
    tsrc = 300
    say(f"gemm tiled algo={algo} fmt={fmt} general={general} amode={amode} R={R}")
    x = synth.random_bf16(92, (tsrc, H))
    gather = dev_i32(np.random.default_rng(93).integers(0, tsrc * 8, size=R).astype(np.int32))
    wg, _ = _gemm_problem(94, E, I, H, counts, tsrc, fmt, general)
    wu, _ = _gemm_problem(95, E, I, H, counts, tsrc, fmt, general)
    wd, _ = _gemm_problem(96, E, D, 2048, counts, R, fmt, general)
    if amode == "nvfp4":
        xc, xs = oracle.quantize_nvfp4(x, 1.0)
        a_dev, a_sc = dev_u8(xc), dev_u8(xs)
    else:
        a_dev, a_sc = dev_bf16(x), None
    z2 = dev_bf16(synth.random_bf16(97, (R, 2048)))
    outs = []
    for tiled in (False, True):
        g, u, d = (moe.tile_weights(w) if tiled else w for w in (wg, wu, wd))
        z = moe.grouped_gemm(a_dev, g, u, offsets, R, gather=gather, gather_div=8, a_scales=a_sc, algo=algo)
        o = moe.grouped_gemm(z2, d, None, offsets, R, algo=algo)
        torch.cuda.synchronize()
        outs.append((host_bf16_bits(z), host_bf16_bits(o)))
    assert np.array_equal(outs[0][0], outs[1][0]), "gate/up differs between layouts"
    assert np.array_equal(outs[0][1], outs[1][1]), "down differs between layouts"


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_grouped_gemm_prefill_narrow_n(fmt):
    """Prefill tiles where N is a multiple of the 128 x 256 tile but not of the
    64 x 512 one (SwiGLU N = 384, down N = 768): ragged experts, bf16 tokens."""
    E, H, I = 8, 768, 384
    counts = np.array(GEMM_COUNTS)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    tsrc = 700
    say(f"gemm prefill narrow-N fmt={fmt} R={R}")
    x = synth.random_bf16(101, (tsrc, H))
    gather = np.random.default_rng(102).integers(0, tsrc * 8, size=R).astype(np.int32)
    wg, dg = _gemm_problem(103, E, I, H, counts, tsrc, fmt)
    wu, du = _gemm_problem(104, E, I, H, counts, tsrc, fmt)
    wd, dd = _gemm_problem(105, E, H, I, counts, R, fmt)
    z = moe.grouped_gemm(dev_bf16(x), wg, wu, dev_i32(offsets), R, gather=dev_i32(gather), gather_div=8,
                         algo=moe.MOE_ALGO_PREFILL)
    z2 = synth.random_bf16(106, (R, I))
    o = moe.grouped_gemm(dev_bf16(z2), wd, None, dev_i32(offsets), R, algo=moe.MOE_ALGO_PREFILL)
    torch.cuda.synchronize()
    a_val, z2v = bf16_to_f64(x), bf16_to_f64(z2)
    zref = np.zeros((R, I))
    oref = np.zeros((R, H))
    for e in range(E):
        rows = slice(offsets[e], offsets[e + 1])
        a = a_val[gather[rows] // 8]
        zref[rows] = oracle.silu(a @ dg[e].T) * (a @ du[e].T)
        oref[rows] = z2v[rows] @ dd[e].T
    zref = bf16_to_f64(oracle.round_to_bf16_bits(zref))
    assert_close_rms(bf16_to_f64(host_bf16_bits(z)), zref, what="z", ulp_rel=BF16_ULP)
    assert_close_rms(bf16_to_f64(host_bf16_bits(o)), oref, what="o", ulp_rel=BF16_ULP)
