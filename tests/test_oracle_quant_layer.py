"""Pins for the oracle's NVFP4 activation quantiser, expert FFN and combine (CPU only)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from oracle.layer import down_proj
from synth import WORKLOADS, activations, bf16_bits_from_f32, expert_weights, logits as gen_logits, random_bf16

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    d = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, *v = line.split()
                d[k] = [float(x) for x in v]
    return d


def _e2m1_table():
    with open(os.path.join(GOLD, "e2m1_magnitudes.txt")) as f:
        return [float(v) for line in f if not line.startswith("#") for v in line.split()]


def test_unit_scale_saturates_at_page_cap():
    g = _golden("activation_outliers.txt")
    cap = g["cap"][0]
    assert cap == 6 * 448
    for amax in g["outlier_amax"] + [cap]:
        x = np.zeros((1, 16), np.float32)
        x[0, 3] = amax
        x[0, 9] = -amax
        x[0, 5] = 1.0
        codes, scales = oracle.quantize_nvfp4(bf16_bits_from_f32(x), 1.0)
        assert scales[0, 0] == 0x7E                           # 448
        v = oracle.dequant_nvfp4_act(codes, scales)
        assert v[0, 3] == cap and v[0, 9] == -cap
        assert v[0, 5] == 0.0                                  # 1/448 rounds to 0 in E2M1


def test_benign_block_is_fine_grained():
    g = _golden("activation_outliers.txt")
    amax = g["benign_amax"][0]
    x = np.linspace(-amax, amax, 16, dtype=np.float32)[None, :]
    codes, scales = oracle.quantize_nvfp4(bf16_bits_from_f32(x), 1.0)
    s = oracle.e4m3_value(scales)[0, 0]
    assert s == 30.0                                           # E4M3(183/6 = 30.5) = 30 (ties to even)


def _brute_block(xs, g):
    table = _e2m1_table()
    e4 = [(Fraction(float(v)), b) for b, v in enumerate(oracle.e4m3_value(np.arange(0x7F)))]
    amax = max(abs(Fraction(float(v))) for v in xs)
    target = min(amax / (6 * Fraction(g)), Fraction(448))
    best = min(e4, key=lambda p: (abs(p[0] - target), p[1] % 2))
    s = best[0]
    nibs = []
    for v in xs:
        fv = Fraction(float(v))
        if s == 0:
            nibs.append(0)
            continue
        r = min(abs(fv) / (s * Fraction(g)), Fraction(6))
        mag = min(range(8), key=lambda i: (abs(r - Fraction(table[i])), i % 2))
        nibs.append(mag | (8 if np.signbit(v) else 0))
    return best[1], nibs


@pytest.mark.parametrize("g", [1.0, 0.5, 4.0])
def test_quantizer_brute_force(g):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((8, 64)) * 10.0 ** rng.integers(-3, 3, (8, 1))).astype(np.float32)
    # exact ties: multiples of a quarter of an E4M3-representable block scale
    x[0, :16] = np.array([6, 5, 4, 3.5, 3, 2.5, 2, 1.75, 1.5, 1.25, 1, .75, .5, .25, 0, -0.0]) * 3.0
    x[1, :16] = 0.0
    x[1, 16:32] = 1e-5                                          # scale rounds to 0
    x[2, 16:32] = -0.0
    xb = bf16_bits_from_f32(x)
    codes, scales = oracle.quantize_nvfp4(xb, g)
    nib = oracle.unpack_codes(codes)
    xv = oracle.bf16_value(xb)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            sb, nibs = _brute_block(xv[r, b * 16:(b + 1) * 16], g)
            assert scales[r, b] == sb, (r, b)
            assert list(nib[r, b * 16:(b + 1) * 16]) == nibs, (r, b)


def test_silu_and_swiglu_closed_form():
    v = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(v), v * expit(v), rtol=1e-14, atol=1e-300)
    # one-hot input picks column j of gate and up: z = silu(Wg[:, j]) * Wu[:, j]
    rng = np.random.default_rng(4)
    wg, wu, wd = rng.standard_normal((3, 64, 32))
    j = 7
    x = np.zeros((1, 32), np.float32)
    x[0, j] = 1.0
    z, o = oracle.expert_ffn(bf16_bits_from_f32(x), wg, wu, wd.T.copy())
    ref = wg[:, j] * expit(wg[:, j]) * wu[:, j]
    assert np.array_equal(z[0], torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)) or \
        np.allclose(oracle.bf16_value(z[0]), ref, rtol=2 ** -8)


def test_gate_up_exact_on_tiny():
    """Tiny shape: the float64 gate/up pre-activations equal exact rational arithmetic."""
    w = WORKLOADS["tiny"]
    x = activations(w, 32)
    W = expert_weights(w)
    table = _e2m1_table()
    for e in range(0, 32, 4):
        wg = oracle.dequant_mx(W["gate"][0][e], W["gate"][1][e])
        got = oracle.bf16_value(x[:4]) @ wg.T
        for t in range(4):
            xs = [Fraction(float(v)) for v in oracle.bf16_value(x[t])]
            for n in range(0, w.shape.inter, 37):
                acc = Fraction(0)
                for k in range(w.shape.hidden):
                    byte = int(W["gate"][0][e, n, k // 2])
                    nib = (byte & 0xF) if k % 2 == 0 else byte >> 4
                    val = Fraction(table[nib & 7]) * (-1 if nib & 8 else 1) * Fraction(2) ** (int(W["gate"][1][e, n, k // 32]) - 127)
                    acc += val * xs[k]
                assert Fraction(float(got[t, n])) == acc


def test_combine_linearity():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((4, 1, 64))
    o = np.repeat(v, 8, axis=1)
    wts = rng.uniform(0.1, 1, (4, 8))
    wts = wts / wts.sum(1, keepdims=True) * 2.827
    y = oracle.combine(o, wts)
    ref = oracle.round_to_bf16_bits(2.827 * v[:, 0, :])
    # sum of weights is 2.827 up to rounding of the float64 weights
    assert np.max(np.abs(oracle.bf16_value(y) - oracle.bf16_value(ref))) <= np.max(np.abs(v)) * 2 ** -7
    res = random_bf16(6, (4, 64))
    y2 = oracle.combine(np.zeros((4, 8, 64)), wts, res)
    assert np.array_equal(y2, res)


def _independent_tiny_layer(x_bits, l, W, s):
    """Straight per-token loops with the golden E2M1 table and torch's E8M0 codec."""
    table = np.array(_e2m1_table())

    def deq(packed, scale):
        nib = np.stack([packed & 0xF, packed >> 4], -1).reshape(packed.shape[0], -1)
        val = table[nib & 7] * np.where(nib & 8, -1.0, 1.0)
        sc = torch.from_numpy(scale.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        return val * np.repeat(sc, 32, axis=1)

    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        ids, wts = _brute(l[t], s)
        for e, wt in zip(ids, wts):
            g = deq(W["gate"][0][e], W["gate"][1][e]) @ x[t]
            u = deq(W["up"][0][e], W["up"][1][e]) @ x[t]
            zf = g * expit(g) * u
            z = torch.from_numpy(zf).to(torch.bfloat16).to(torch.float64).numpy()
            y[t] += wt * (deq(W["down"][0][e], W["down"][1][e]) @ z)
    return y


def _brute(lt, s):
    sg = expit(lt.astype(np.float64))
    gs = s.num_experts // s.n_group
    gsc = [np.sort(sg[g * gs:(g + 1) * gs])[-2:].sum() for g in range(s.n_group)]
    kept = sorted(range(s.n_group), key=lambda g: (-gsc[g], g))[:s.topk_group]
    cand = sorted([e for g in kept for e in range(g * gs, (g + 1) * gs)], key=lambda e: (-sg[e], e))[:s.top_k]
    w = sg[cand]
    return cand, w / w.sum() * s.routed_scaling_factor


def test_tiny_layer_against_independent_loops():
    w = WORKLOADS["tiny"]
    s = w.shape
    x = activations(w, 32)
    l = gen_logits(w, 32)
    W = expert_weights(w)
    res = oracle.moe_layer(x, l, None, W, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
    ref = _independent_tiny_layer(x, l, W, s)
    got = oracle.bf16_value(res.y)
    # z goes through a float64->float32->bf16 double rounding in torch above; allow an ulp of z
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(got - ref)) <= 2e-3 * rms + np.max(np.abs(ref)) * 2 ** -8


def _fake_quant_brute(v):
    """NVFP4 quantise-dequantise of float64 values (bf16-exact) with the brute-force rules above."""
    table = _e2m1_table()
    out = np.empty_like(v)
    e4 = oracle.e4m3_value(np.arange(0x7F))
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 16):
            blk = v[r, b * 16:(b + 1) * 16]
            sb, nibs = _brute_block(blk, 1.0)
            out[r, b * 16:(b + 1) * 16] = [table[n & 7] * (-1 if n & 8 else 1) * e4[sb] for n in nibs]
    return out


def test_tiny_w4a4_layer_against_brute_force():
    """W4A4 on the tiny shape: x and z both fake-quantised by the brute-force rules."""
    w = WORKLOADS["tiny"]
    s = w.shape
    T = 6
    x = activations(w, 32)[:T]
    l = gen_logits(w, 32)[:T]
    W = expert_weights(w)
    nv = {}
    for name in ("gate", "up", "down"):
        sc, g, _ = oracle.transcode_mx_to_nv(W[name][1], W[name][0])
        nv[name] = (W[name][0], sc, g)
    res = oracle.moe_layer(x, l, None, nv, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor,
                           fmt="nv", act_mode="nvfp4")
    xq = _fake_quant_brute(oracle.bf16_value(x))
    y = np.zeros((T, s.hidden))
    for t in range(T):
        ids, wts = _brute(l[t], s)
        for j, (e, wt) in enumerate(zip(ids, wts)):
            wg = oracle.dequant_mx(W["gate"][0][e], W["gate"][1][e])
            wu = oracle.dequant_mx(W["up"][0][e], W["up"][1][e])
            wd = oracle.dequant_mx(W["down"][0][e], W["down"][1][e])
            g = wg @ xq[t]
            u = wu @ xq[t]
            z = oracle.bf16_value(oracle.round_to_bf16_bits(g * expit(g) * u))
            assert np.array_equal(oracle.round_to_bf16_bits(z), res.z[t, j]) or \
                np.max(np.abs(z - oracle.bf16_value(res.z[t, j]))) <= np.max(np.abs(z)) * 2 ** -7
            zq = _fake_quant_brute(oracle.bf16_value(res.z[t, j])[None, :])[0]
            y[t] += wt * (wd @ zq)
    got = oracle.bf16_value(res.y)
    assert np.max(np.abs(got - y)) <= np.max(np.abs(y)) * 2 ** -8


# ------------------------------------------------------------------ MXFP8
def _mxfp8_input(seed=31, rows=67, k=256):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, k)) * 10.0 ** rng.integers(-6, 6, (rows, 1))).astype(np.float32)
    x[0, :32] = 0.0                              # an all-zero block
    x[0, 32:64] = -0.0                           # negative zeros
    x[1, :32] = 1.0
    x[1, 5] = 2.0 ** 7                           # amax a power of two: maps to exactly 256
    x[2, :32] = 0.5
    x[2, 0] = 1.75 * 2 ** 3                      # amax / X = 448 exactly
    x[3, :32] = 0.25
    x[3, 0] = 1.875 * 2 ** 3                     # amax / X = 480: saturates at 448
    x[4, :32] = 2.0 ** -20
    x[4, 0] = 1.0                                # small elements fall into E4M3 subnormals or to zero
    return bf16_bits_from_f32(x)


def test_mxfp8_codes_match_torch_float8_codec():
    """Codes are torch's float8_e4m3fn rounding (nearest-even) of x / X after
    clamping to +-448; scales are E8M0 powers of two; the zero sign follows x."""
    xb = _mxfp8_input()
    codes, scales = oracle.quantize_mxfp8(xb)
    x = oracle.bf16_value(xb)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    q = np.clip(x / X, -448.0, 448.0)
    ref = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # torch's float8 decode agrees with the oracle's dequantisation
    back = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64) * X
    assert np.array_equal(oracle.dequant_mxfp8(codes, scales), back)


def test_mxfp8_scale_rule_properties():
    """max|x| / X lies in [256, 512) for every non-zero block (the scale is the
    power of two that puts the block maximum in E4M3's top binade or saturates
    it), a zero block gets 2^-127, and the worked cases land where the format says."""
    xb = _mxfp8_input()
    codes, scales = oracle.quantize_mxfp8(xb)
    x = oracle.bf16_value(xb).reshape(xb.shape[0], -1, 32)
    amax = np.abs(x).max(axis=-1)
    X = np.ldexp(1.0, scales.astype(np.int64) - 127)
    nz = amax > 0
    r = amax[nz] / X[nz]
    assert np.all((r >= 256) & (r < 512))
    assert np.all(scales[~nz] == 0)
    c = codes.reshape(xb.shape[0], -1, 32)
    assert np.all(c[0, 0] == 0) and np.all(c[0, 1] == 0x80)          # +0 and -0 blocks
    assert c[1, 0, 5] == 0x78 and scales[1, 0] == 127 + 7 - 8        # 2^7 -> 256 * 2^-1
    assert c[2, 0, 0] == 0x7E                                        # 448
    assert c[3, 0, 0] == 0x7E                                        # 480 saturates at 448
    v = oracle.dequant_mxfp8(codes, scales).reshape(x.shape)
    assert v[3, 0, 0] == 448 * 2.0 ** -5
    # 2^-20 with X = 2^-8: 2^-12 < half of E4M3's smallest subnormal 2^-9 -> 0
    assert np.all(c[4, 0, 1:] == 0)


def test_mxfp8_brute_force_nearest():
    """Every code is the nearest E4M3 value to x / X (ties to the even code),
    found by search over all 126 finite magnitudes, unless |x / X| > 448."""
    xb = random_bf16(33, (16, 128), std=3.0)
    codes, scales = oracle.quantize_mxfp8(xb)
    x = oracle.bf16_value(xb)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    grid = [(Fraction(oracle.e4m3_value(b).item()), b) for b in range(0x7F)]
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            t = abs(Fraction(x[i, j]) / Fraction(X[i, j]))
            if t > 448:
                want = 0x7E
            else:
                best = min(grid, key=lambda gb: (abs(gb[0] - t), gb[1] & 1))
                want = best[1]
            want |= 0x80 if np.signbit(x[i, j]) else 0
            assert codes[i, j] == want, (i, j, x[i, j], codes[i, j], want)


# ----------------------------------------------------------- REAP saliency
def test_saliency_worked_example():
    """Two tokens, top-2 of 3 experts, outputs with known norms (3-4-5 rows):
    S_0 = (0.5 * 5 + 0.25 * 13) / 2, S_1 = 0.5 * 10, S_2 = 0.75 * 13, and S_j
    is unchanged when the same batch is accumulated twice."""
    o = np.zeros((2, 2, 4))
    o[0, 0, :2] = [3, 4]          # token 0 -> expert 0, norm 5
    o[0, 1, :2] = [6, 8]          # token 0 -> expert 1, norm 10
    o[1, 0, 1:4] = [3, 4, 12]     # token 1 -> expert 2, norm 13
    o[1, 1, 1:4] = [3, 4, 12]     # token 1 -> expert 0, norm 13
    ids = np.array([[0, 1], [2, 0]])
    g = np.array([[0.5, 0.5], [0.75, 0.25]])
    sums, counts = oracle.saliency_accumulate(o, g, ids, 3)
    np.testing.assert_array_equal(counts, [2, 1, 1])
    np.testing.assert_allclose(oracle.saliency(sums, counts), [(2.5 + 3.25) / 2, 5.0, 9.75], rtol=1e-15)
    sums2, counts2 = oracle.saliency_accumulate(o, g, ids, 3, sums.copy(), counts.copy())
    np.testing.assert_allclose(oracle.saliency(sums2, counts2), oracle.saliency(sums, counts), rtol=1e-15)


def test_saliency_equal_outputs_closed_form():
    """Every expert output equal to v: S_j = mean of g over j's tokens x ||v||;
    an expert no token reached has no saliency (NaN)."""
    rng = np.random.default_rng(3)
    T, k, E, H = 50, 4, 9, 16
    v = rng.standard_normal(H)
    ids = np.stack([rng.permutation(E - 1)[:k] for _ in range(T)])        # expert E-1 never routed
    g = rng.uniform(0.1, 1.0, (T, k))
    o = np.broadcast_to(v, (T, k, H))
    S = oracle.saliency(*oracle.saliency_accumulate(o, g, ids, E))
    for e in range(E - 1):
        np.testing.assert_allclose(S[e], g[ids == e].mean() * np.linalg.norm(v), rtol=1e-13)
    assert np.isnan(S[E - 1])


def test_down_proj_against_exact_rationals():
    """down_proj contracts z [m, I] with W_down [H, I] over I (o = z W_downᵀ, the
    outer W_down of the REAP saliency equation): each float64 output lies within
    the float64 summation bound of the exact rational sum of its terms, and an
    operand transposed or a term dropped fails the check."""
    w = WORKLOADS["tiny"]
    W = expert_weights(w)
    table = _e2m1_table()
    z = random_bf16(41, (3, w.shape.inter), std=0.5)
    zs = oracle.bf16_value(z)
    I = w.shape.inter
    for e in (0, 13, 31):
        wd = oracle.dequant_mx(W["down"][0][e], W["down"][1][e])
        assert wd.shape == (w.shape.hidden, I)
        got = down_proj(z, wd)
        assert got.shape == (3, w.shape.hidden)
        for t in range(3):
            zf = [Fraction(float(v)) for v in zs[t]]
            for n in range(0, w.shape.hidden, 29):
                acc, mag = Fraction(0), Fraction(0)
                for k in range(I):
                    byte = int(W["down"][0][e, n, k // 2])
                    nib = (byte & 0xF) if k % 2 == 0 else byte >> 4
                    val = Fraction(table[nib & 7]) * (-1 if nib & 8 else 1) * \
                        Fraction(2) ** (int(W["down"][1][e, n, k // 32]) - 127)
                    acc += val * zf[k]
                    mag += abs(val * zf[k])
                assert abs(Fraction(float(got[t, n])) - acc) <= I * Fraction(2) ** -53 * mag


def test_down_proj_nvfp4_on_exactly_representable_z():
    """A z whose every 16-value block is E2M1 values times one power of two the
    E4M3 scale can hold is quantised to NVFP4 without loss, so the W4A4 down
    projection equals the bf16 one on it; the same z perturbed by one bf16 ulp
    in one element is not representable and the results differ."""
    rng = np.random.default_rng(43)
    table = np.array(_e2m1_table())
    I, H = 64, 48
    mags = table[rng.integers(0, 8, (2, I))] * np.where(rng.random((2, I)) < 0.5, -1.0, 1.0)
    mags[:, ::16] = 6.0                        # every block reaches the E2M1 maximum
    scale = 2.0 ** rng.integers(-4, 4, (2, I // 16)).repeat(16, axis=1)
    z = bf16_bits_from_f32((mags * scale).astype(np.float32))
    wd = rng.standard_normal((H, I))
    ref = down_proj(z, wd)
    np.testing.assert_array_equal(down_proj(z, wd, act_mode="nvfp4"), ref)
    z2 = z.copy()
    z2[0, 5] = np.uint16(int(z2[0, 5]) + 1) if mags[0, 5] != 0 else np.uint16(0x3F81)
    assert not np.array_equal(down_proj(z2, wd, act_mode="nvfp4"), down_proj(z2, wd))
