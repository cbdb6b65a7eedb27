"""Compact MXFP4 expert storage (4.125 bits per weight) on the GPU.

The converter is integer work: its exponent codes, bases and counters must
equal the oracle's byte for byte.  A GEMM on lossless compact weights computes
with the same values as on the MXFP4 weights they came from; the kernel folds
the matrix base (a power of two) into the epilogue, which scales every product
by one power of two and leaves each rounding where it was, so the outputs are
bit-identical to the MXFP4 path's (and the MXFP4 path is checked against the
oracle elsewhere).  One case also goes to the oracle directly, through its
compact dequantisation.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_ULP, assert_close_rms, bf16_to_f64, dev_bf16, dev_i32, dev_u8, host, host_bf16_bits, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import block_scaled_fp4_group_amd as moe  # noqa: E402


def _convert_case(mx, packed):
    c_ref, b_ref, cnt_ref = oracle.compact_mx(mx, packed)
    c, b, cnt = moe.compact_mx(dev_u8(mx), dev_u8(packed))
    torch.cuda.synchronize()
    assert np.array_equal(host(c), c_ref)
    assert np.array_equal(host(b).view(np.uint32), b_ref.view(np.uint32))
    got = list(host(cnt))
    assert got == [cnt_ref["blocks"], cnt_ref["zero_oor"], cnt_ref["rerounded"], cnt_ref["nan"]], got
    return got


def test_compact_converter_parity_random():
    say("compact converter: random MXFP4, 12 x [64, 1024]")
    packed, mx = synth.random_mx_small(121, 12, 64, 1024)
    cnt = _convert_case(mx, packed)
    assert cnt[1:] == [0, 0, 0]


def test_compact_converter_parity_edge_blocks():
    """Spans beyond 15, NaN scales, an all-zero block below the window, a
    matrix with no finite block, E8M0 0 and 254."""
    say("compact converter: edge blocks")
    packed, mx = synth.random_mx_small(122, 6, 32, 512, lo=100, hi=140)
    mx, packed = mx.copy(), packed.copy()
    mx[0, 0, 0] = 200                  # span 100: many blocks below the window
    mx[1, 3, 2] = 255                  # NaN
    mx[2, :, :] = 127
    mx[2, 0, 0] = 127 + 15             # span 15 exactly: every block representable
    mx[2, 5, 1] = 0                    # 2^-127 below the window ...
    packed[2, 5, 16:32] = 0x80         # ... with all -0 codes: exact
    mx[3] = 255                        # no finite block: base 1
    mx[4, :, :] = 127
    mx[4, 0, 0] = 127 + 16             # span 16: blocks at 127 are re-rounded
    mx[5, :, :] = 254                  # largest finite E8M0
    mx[5, 1, 3] = 0
    cnt = _convert_case(mx, packed)
    assert cnt[1] >= 1 and cnt[2] >= 1 and cnt[3] >= 32 * 16 + 1


def test_compact_converter_model_shape():
    """Expert matrices at the model's [2048, 4096] / [4096, 2048]: lossless."""
    w = synth.WORKLOADS["decode"]
    W = synth.expert_weights(w, experts=[0, 1, 2])
    for name in ("gate", "down"):
        say(f"compact converter: model {name}")
        packed, mx = W[name]
        cnt = _convert_case(mx, packed)
        assert cnt[1:] == [0, 0, 0]


def test_compact_tile_layout():
    """Tiled compact scales: 16 rows x 8 bytes per 512-column window."""
    E, n, k = 3, 48, 1536
    say(f"compact tile layout E={E} n={n} k={k}")
    rng = np.random.default_rng(123)
    codes = rng.integers(0, 256, size=(E, n, k // 2), dtype=np.uint8)
    sc = rng.integers(0, 256, size=(E, n, k // 64), dtype=np.uint8)
    base = torch.ones(E, dtype=torch.float32, device="cuda")
    w = moe.tile_weights(moe.Weights(dev_u8(codes), dev_u8(sc), base, compact=True))
    torch.cuda.synchronize()
    c = codes.reshape(E, n // 16, 16, k // 128, 4, 16).transpose(0, 1, 3, 4, 2, 5).reshape(codes.shape)
    s = sc.reshape(E, n // 16, 16, k // 512, 8).transpose(0, 1, 3, 2, 4).reshape(sc.shape)
    assert w.tiled and w.compact
    assert np.array_equal(host(w.packed), c)
    assert np.array_equal(host(w.scale), s)


def _mx_weights(seed, E, n, k):
    packed, mx = synth.random_mx_small(seed, E, n, k)
    return moe.Weights(dev_u8(packed), dev_u8(mx)), packed, mx


# (experts, gate/up rows, down rows, row counts): K split in 4 with many 8-row
# passes or single rows; 64 experts: whole K per wave (two tiles per gate/up
# wave, eight waves per down workgroup)
CASES = {
    "ragged": (8, 512, 512, [0, 1, 17, 150, 400, 33, 0, 64]),
    "single": (8, 512, 512, [1, 0, 1, 1, 0, 0, 1, 1]),
    "wide": (64, 1024, 2048, None),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("amode", ["bf16", "nvfp4"])
def test_compact_gemm_is_bitwise_mx(case, tiled, amode):
    E, I, D, counts = CASES[case]
    H = 4096
    if counts is None:
        counts = list(np.random.default_rng(124).integers(0, 9, size=E))
    counts = np.array(counts)
    offsets = dev_i32(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    R = int(counts.sum())
    tsrc = max(R, 8)
    say(f"compact gemm case={case} tiled={tiled} amode={amode} E={E} R={R}")
    x = synth.random_bf16(125, (tsrc, H))
    gather = dev_i32(np.random.default_rng(126).integers(0, tsrc * 8, size=R).astype(np.int32))
    wg, _, _ = _mx_weights(127, E, I, H)
    wu, _, _ = _mx_weights(128, E, I, H)
    wd, _, _ = _mx_weights(129, E, D, 2048)
    if amode == "nvfp4":
        xc, xs = oracle.quantize_nvfp4(x, 1.0)
        a_dev, a_sc = dev_u8(xc), dev_u8(xs)
    else:
        a_dev, a_sc = dev_bf16(x), None
    z2 = dev_bf16(synth.random_bf16(130, (R, 2048)))
    outs = []
    for compact in (False, True):
        ws = []
        for w in (wg, wu, wd):
            if compact:
                w, cnt = moe.compact_weights(w)
                torch.cuda.synchronize()
                assert list(host(cnt)[1:]) == [0, 0, 0]
            ws.append(moe.tile_weights(w) if tiled else w)
        g, u, d = ws
        z = moe.grouped_gemm(a_dev, g, u, offsets, R, gather=gather, gather_div=8, a_scales=a_sc,
                             algo=moe.MOE_ALGO_DECODE)
        o = moe.grouped_gemm(z2, d, None, offsets, R, algo=moe.MOE_ALGO_DECODE)
        torch.cuda.synchronize()
        outs.append((host_bf16_bits(z), host_bf16_bits(o)))
    assert np.array_equal(outs[0][0], outs[1][0]), "gate/up: compact differs from MXFP4"
    assert np.array_equal(outs[0][1], outs[1][1]), "down: compact differs from MXFP4"


def test_compact_gemm_against_oracle():
    """The compact GEMM against the oracle's own compact dequantisation, at a
    K the unrolled kernels do not cover (1536: the runtime step loop)."""
    E, H, I = 4, 1536, 256
    counts = np.array([5, 0, 23, 9])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    say(f"compact gemm vs oracle E={E} H={H} I={I} R={R}")
    x = synth.random_bf16(131, (R, H))
    mats = []
    for seed in (132, 133):
        packed, mx = synth.random_mx_small(seed, E, I, H)
        c4, base, cnt = oracle.compact_mx(mx, packed)
        assert cnt["rerounded"] == 0 and cnt["nan"] == 0
        dq = [oracle.dequant_compact(packed[e], c4[e], base[e]) for e in range(E)]
        w = moe.Weights(dev_u8(packed), dev_u8(c4), torch.from_numpy(base).cuda(), compact=True)
        mats.append((w, dq))
    (wg, dg), (wu, du) = mats
    z = moe.grouped_gemm(dev_bf16(x), wg, wu, dev_i32(offsets), R)
    torch.cuda.synchronize()
    xv = bf16_to_f64(x)
    ref = np.zeros((R, I))
    for e in range(E):
        rows = slice(offsets[e], offsets[e + 1])
        ref[rows] = oracle.silu(xv[rows] @ dg[e].T) * (xv[rows] @ du[e].T)
    ref = bf16_to_f64(oracle.round_to_bf16_bits(ref))
    assert_close_rms(bf16_to_f64(host_bf16_bits(z)), ref, what="z (compact)", ulp_rel=BF16_ULP)


def test_compact_gemm_rejects_prefill_only_requests():
    w, _, _ = _mx_weights(134, 4, 256, 512)
    wc, _ = moe.compact_weights(w)
    offs = dev_i32(np.array([0, 2, 2, 2, 2], np.int32))
    x = dev_bf16(synth.random_bf16(135, (2, 512)))
    with pytest.raises(moe.MoeError) as ei:
        moe.grouped_gemm(x, wc, None, offs, 2, algo=moe.MOE_ALGO_PREFILL)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        moe.compact_weights(moe.tile_weights(w))


@pytest.fixture(scope="module")
def decode_layer_weights():
    """Decode-shape weights in the tiled layout: MXFP4, and the same in compact storage."""
    from test_gpu_layer import upload_weights
    dw = upload_weights(synth.expert_weights(synth.WORKLOADS["decode"]), "mx")
    mx = moe.LayerWeights(*(moe.tile_weights(getattr(dw, n)) for n in ("gate", "up", "down")))
    cw = []
    for n in ("gate", "up", "down"):
        c, cnt = moe.compact_weights(getattr(dw, n))
        torch.cuda.synchronize()
        assert list(host(cnt)[1:]) == [0, 0, 0]
        cw.append(moe.tile_weights(c))
    return mx, moe.LayerWeights(*cw)


@pytest.mark.parametrize("T", [1, 8, 64])
def test_compact_decode_layer_is_bitwise_mx(decode_layer_weights, T):
    """The whole decode layer (route, permute, both GEMMs, combine) on compact
    tiled weights gives the bytes of the layer on the MXFP4 weights, from a HIP
    graph replayed with new inputs (eager work between the replays)."""
    w = synth.WORKLOADS["decode"]
    s = w.shape
    mx, cw = decode_layer_weights
    mk = lambda lw: moe.MoELayer(lw, s.num_experts, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor, T)
    lay_mx, lay_c = mk(mx), mk(cw)
    x_static = dev_bf16(synth.activations(w, T))
    l_static = torch.from_numpy(synth.logits(w, T)).cuda()
    y_static = torch.empty((T, s.hidden), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lay_c.forward(x_static, l_static, y=y_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lay_c.forward(x_static, l_static, y=y_static)
    torch.cuda.synchronize()
    rng = np.random.default_rng(29)
    for rep in range(3):
        say(f"compact layer T={T} rep={rep}")
        xb = synth.bf16_bits_from_f32(rng.standard_normal((T, s.hidden)).astype(np.float32))
        lg = rng.standard_normal((T, s.num_experts)).astype(np.float32)
        x_new, l_new = dev_bf16(xb), torch.from_numpy(lg).cuda()
        x_static.copy_(x_new)
        l_static.copy_(l_new)
        graph.replay()
        torch.cuda.synchronize()
        y_mx = host_bf16_bits(lay_mx.forward(x_new, l_new)).copy()
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16_bits(y_static), y_mx), f"replay {rep}: compact layer differs from MXFP4"
