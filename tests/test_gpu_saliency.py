"""GPU parity of the REAP saliency accumulation (down-projection epilogue sums
of squares, then a per-expert reduction) against the oracle.

Step-wise: the oracle takes the GPU's own bf16 z, computes the float64 expert
outputs, and accumulates g ||o|| per expert; the GPU's parts of ||o||^2 come
from its FP32 accumulators, so the figures agree to FP32 accumulation error
(rtol 1e-5).  The per-row parts are checked against the oracle's float64 ones
too, and the whole computation gives the same bits twice.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_to_f64, dev_bf16, dev_f32, dev_i32, dev_u8, host, host_bf16_bits, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_group_amd as moe  # noqa: E402


@pytest.mark.parametrize("tiled", [False, True])
def test_row_sumsq_and_saliency_kernel(tiled):
    E, H, I = 16, 1024, 512
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 400, E)
    counts[3] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    T = (R + 7) // 8
    say(f"saliency kernel tiled={tiled} R={R}")
    z = synth.random_bf16(401, (R, I))
    packed, mx = synth.random_mx_small(402, E, H, I)
    w = moe.Weights(dev_u8(packed), dev_u8(mx))
    if tiled:
        w = moe.tile_weights(w)
    sq = torch.full((R, H // 64), -1.0, dtype=torch.float32, device="cuda")
    o = moe.grouped_gemm(dev_bf16(z), w, None, dev_i32(offsets), R, row_sumsq=sq)
    slots = rng.permutation(T * 8)[:R].astype(np.int32)          # a permutation's sorted slots
    topw = rng.uniform(0.05, 0.6, T * 8).astype(np.float32)
    sums = torch.zeros(E, dtype=torch.float64, device="cuda")
    cnts = torch.zeros(E, dtype=torch.int64, device="cuda")
    for _ in range(2):                                            # two batches accumulate
        moe.reap_saliency_accumulate(sq, dev_i32(offsets), dev_i32(slots), dev_f32(topw), sums, cnts, R)
    torch.cuda.synchronize()
    zv = bf16_to_f64(z)
    o64 = np.zeros((R, H))
    for e in range(E):
        r = slice(offsets[e], offsets[e + 1])
        o64[r] = zv[r] @ oracle.dequant_mx(packed[e], mx[e]).T
    parts = (o64 ** 2).reshape(R, H // 64, 64).sum(axis=-1)
    np.testing.assert_allclose(host(sq), parts, rtol=1e-5)
    # the oracle on the same rows: ids and weights in slot order
    ids = np.full(T * 8, -1)
    g = np.zeros(T * 8)
    rows_of_slot = np.full(T * 8, -1)
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            ids[slots[r]] = e
            g[slots[r]] = topw[slots[r]]
            rows_of_slot[slots[r]] = r
    used = ids >= 0
    o_slots = o64[rows_of_slot[used]][None]
    s_ref, c_ref = oracle.saliency_accumulate(o_slots, g[used][None].astype(np.float64), ids[used][None], E)
    s_ref, c_ref = 2 * s_ref, 2 * c_ref
    np.testing.assert_array_equal(host(cnts), c_ref)
    np.testing.assert_allclose(host(sums), s_ref, rtol=1e-5)
    # deterministic: the same call again gives the same bits
    sums2 = torch.zeros(E, dtype=torch.float64, device="cuda")
    cnts2 = torch.zeros(E, dtype=torch.int64, device="cuda")
    for _ in range(2):
        moe.reap_saliency_accumulate(sq, dev_i32(offsets), dev_i32(slots), dev_f32(topw), sums2, cnts2, R)
    torch.cuda.synchronize()
    assert np.array_equal(host(sums).view(np.int64), host(sums2).view(np.int64))


def test_reap_layer_saliency_two_batches():
    """The REAP-50 layer shape (128 experts, Zipf routing), two batches of 2048
    tokens through MoELayer(saliency=True): S step-wise against the oracle on the
    GPU's own z, and end to end against the oracle's layer (reported)."""
    w = synth.WORKLOADS["reap50"]
    s = w.shape
    W = synth.expert_weights(w)
    from test_gpu_layer import ExpertCache, upload_weights
    dw = upload_weights(W, "mx")
    T = 2048
    layer = moe.MoELayer(dw, s.num_experts, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor, T,
                         keep_z_bf16=True, saliency=True)
    cache = ExpertCache(W, "mx")
    s_ref = np.zeros(s.num_experts)
    c_ref = np.zeros(s.num_experts, np.int64)
    for b in range(2):
        say(f"REAP saliency batch {b}")
        x = synth.activations(w, T, b)
        l = synth.logits(w, T, b)
        layer.forward(dev_bf16(x), dev_f32(l))
        torch.cuda.synchronize()
        R = T * s.top_k
        z = host_bf16_bits(layer.z[:R])
        off, ss = host(layer.offsets), host(layer.sorted_slots[:R])
        topw = host(layer.topw[:T]).reshape(-1).astype(np.float64)
        ids = host(layer.ids[:T]).reshape(-1)
        for e in range(s.num_experts):
            r0, r1 = int(off[e]), int(off[e + 1])
            if r1 == r0:
                continue
            o = bf16_to_f64(z[r0:r1]) @ cache(e)[2].T
            sl = ss[r0:r1]
            assert np.all(ids[sl] == e)
            s_ref, c_ref = oracle.saliency_accumulate(o[None], topw[sl][None], ids[sl][None], s.num_experts,
                                                      s_ref, c_ref)
    np.testing.assert_array_equal(host(layer.sal_counts), c_ref)
    S_gpu = oracle.saliency(host(layer.sal_sums), host(layer.sal_counts))
    S_ref = oracle.saliency(s_ref, c_ref)
    seen = c_ref > 0
    np.testing.assert_allclose(S_gpu[seen], S_ref[seen], rtol=1e-5)
    say(f"  experts reached {int(seen.sum())} of {s.num_experts}; S range {np.nanmin(S_gpu):.4e} .. {np.nanmax(S_gpu):.4e}")
