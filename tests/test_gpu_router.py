"""GPU parity of the router matmul and its group top-k (moe_route_gemv)
against the oracle's float64 router matmul and routing, through the C ABI.

ids exactly on every token (and no token of these workloads has a decision
within 1e-12 of a tie), weights to rtol 1e-6, the float64 logits within the
float64 summation bound of the oracle's.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_group_amd as moe  # noqa: E402

# T <= 16 runs the one-workgroup-per-expert kernel (1, <= 8 and <= 16 tokens per
# thread), larger T the 16 x 16 MFMA tiles
CASES = [("tiny", 32, False), ("tiny", 5, False), ("tiny", 3, False), ("decode", 1, False), ("decode", 8, False),
         ("decode", 16, False), ("prefill", 13, True), ("decode", 64, False), ("decode", 67, False),
         ("prefill", 8192, True), ("reap50", 4096, False)]


@pytest.mark.parametrize("name,T,with_bias", CASES)
def test_route_gemv_parity(name, T, with_bias):
    w = synth.WORKLOADS[name]
    s = w.shape
    say(f"route_gemv {name} T={T}")
    x = synth.activations(w, T)
    W = synth.router_weight(w)
    bias = synth.correction_bias(w) if with_bias else None
    r, l_ref = oracle.route_hidden(x, W, bias, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
    ws = torch.full((moe.route_gemv_workspace_bytes(T, s.num_experts),), 0xA5, dtype=torch.uint8, device="cuda")
    xd, Wd, bd = dev_bf16(x), dev_f32(W), None if bias is None else dev_f32(bias)
    for rep in range(2):                       # a second call on the same workspace
        ids, wts = moe.route_gemv(xd, Wd, bd, s.num_experts, s.n_group, s.topk_group, s.top_k,
                                  s.routed_scaling_factor, ws)
        torch.cuda.synchronize()
        say(f"  rep {rep}: near-ties flagged {int(r.near_tie.sum())}")
        assert not r.near_tie.any()
        assert np.array_equal(host(ids), r.ids)
        np.testing.assert_allclose(host(wts), r.weights, rtol=1e-6)
        wsh = host(ws)
        n = T * s.num_experts
        logits = wsh[:n * 8].view(np.float64).reshape(T, s.num_experts)
        mag = oracle.bf16_value(x).__abs__() @ np.abs(W.astype(np.float64)).T
        bound = 2 * s.hidden * 2.0 ** -53 * mag
        assert np.all(np.abs(logits - l_ref) <= bound)


def test_route_gemv_rejects():
    w = synth.WORKLOADS["decode"]
    s = w.shape
    x = torch.zeros((4, 768), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((256, 768), dtype=torch.float32, device="cuda")
    ws = torch.zeros(moe.route_gemv_workspace_bytes(4, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:                 # hidden must be a multiple of 512
        moe.route_gemv(x, W, None, 256, 8, 4, 8, 2.827, ws)
    assert ei.value.status == moe.MOE_ERR_INVALID
    x = torch.zeros((4, 4096), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((256, 4096), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.route_gemv(x, W, None, 256, 8, 4, 8, 2.827, ws[:16])
    assert ei.value.status == moe.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("T", [1, 64])
def test_decode_layer_with_router_matmul(T):
    """The decode layer run from hidden states alone (router matmul fused with
    the top-k, then the permutation): routing, permutation and y against the
    oracle on the same float64 logits."""
    w = synth.WORKLOADS["decode"]
    s = w.shape
    from test_gpu_layer import upload_weights, ExpertCache
    W = synth.expert_weights(w)
    dw = upload_weights(W, "mx")
    x = synth.activations(w, T)
    RW = synth.router_weight(w)
    layer = moe.MoELayer(dw, s.num_experts, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor, T,
                         router_weight=dev_f32(RW))
    y = layer.forward(dev_bf16(x), None)
    torch.cuda.synchronize()
    r, l64 = oracle.route_hidden(x, RW, None, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
    assert not r.near_tie.any()
    assert np.array_equal(host(layer.ids[:T]), r.ids)
    off, ss, sr = oracle.permute(r.ids, s.num_experts)
    assert np.array_equal(host(layer.offsets), off)
    assert np.array_equal(host(layer.sorted_slots[:T * s.top_k]), ss)
    # the expert FFNs and combine on the oracle's routing of the same logits
    cache = ExpertCache(W, "mx")
    toks = np.arange(min(T, 4))
    o = np.zeros((len(toks), s.top_k, s.hidden))
    for i, t in enumerate(toks):
        for j in range(s.top_k):
            wg, wu, wd = cache(int(r.ids[t, j]))
            _, o[i, j] = oracle.expert_ffn(x[t:t + 1], wg, wu, wd)
    y64 = oracle.combine_f64(o, r.weights[toks])
    from gpu_util import assert_close_rms, bf16_to_f64, host_bf16_bits
    assert_close_rms(bf16_to_f64(host_bf16_bits(y)[toks]), y64, what="y (end-to-end, literal)")


@pytest.mark.parametrize("T", [1, 64])
def test_router_layer_hip_graph(T):
    """The decode layer with the router matmul captured in a HIP graph: every
    replay (new hidden states copied into the captured buffer, eager work and
    synchronisations between replays) gives the bytes of an eager forward."""
    w = synth.WORKLOADS["decode"]
    s = w.shape
    from test_gpu_layer import upload_weights
    dw = upload_weights(synth.expert_weights(w), "mx")
    RW = dev_f32(synth.router_weight(w))
    mk = lambda: moe.MoELayer(dw, s.num_experts, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor, T,
                              router_weight=RW)
    layer, eager = mk(), mk()
    x_static = dev_bf16(synth.activations(w, T))
    y_static = torch.empty((T, s.hidden), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x_static, None, y=y_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(x_static, None, y=y_static)
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    from gpu_util import host_bf16_bits
    for rep in range(4):
        say(f"router graph replay T={T} rep={rep}")
        xb = synth.bf16_bits_from_f32(rng.standard_normal((T, s.hidden)).astype(np.float32))
        x_new = dev_bf16(xb)
        x_static.copy_(x_new)
        graph.replay()
        torch.cuda.synchronize()
        y_ref = host_bf16_bits(eager.forward(x_new, None)).copy()
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16_bits(y_static), y_ref), f"replay {rep} differs from eager"
        assert np.array_equal(host(layer.ids[:T]), host(eager.ids[:T]))
