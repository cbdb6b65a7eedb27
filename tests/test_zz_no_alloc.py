"""moe_route_permute_noalloc (static scratch, no allocation) against
moe_route_permute (caller counter and workspace): identical bytes on two calls
in a row, the second smaller, on both of its paths (one fused launch up to
2048 slots, separate router and permutation launches above)."""
import numpy as np
import pytest

import synth
from gpu_util import dev_f32, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_group_amd as moe  # noqa: E402


def _outputs(T, E, top_k):
    i32 = torch.int32
    return (torch.full((T, top_k), -5, dtype=i32, device="cuda"),
            torch.full((T, top_k), -5.0, dtype=torch.float32, device="cuda"),
            torch.full((E + 1,), -5, dtype=i32, device="cuda"),
            torch.full((T * top_k,), -5, dtype=i32, device="cuda"),
            torch.full((T * top_k,), -5, dtype=i32, device="cuda"))


@pytest.mark.parametrize("sizes", [(4096, 64), (64, 1), (9000, 3000)])
def test_noalloc_matches_route_permute(sizes):
    E, n_group, topk_group, top_k = 256, 8, 4, 8
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(sum(sizes))
    bias = dev_f32((rng.standard_normal(E) * 0.3).astype(np.float32))
    for call, T in enumerate(sizes):
        say(f"noalloc call {call}: T={T} (R={T * top_k})")
        l = dev_f32(synth.random_logits(1000 + T, T, E))
        ref = moe.route_permute(l, bias, E, n_group, topk_group, top_k, 2.827, counter)
        got = moe.route_permute_noalloc(l, bias, E, n_group, topk_group, top_k, 2.827, *_outputs(T, E, top_k))
        torch.cuda.synchronize()
        for name, a, b in zip(("ids", "weights", "offsets", "sorted_slots", "slot_rows"), ref, got):
            assert np.array_equal(host(a).view(np.int32), host(b).view(np.int32)), f"{name} differs (T={T})"


def test_noalloc_rejects_oversize():
    E, top_k = 256, 8
    T = (1 << 27) // (E * top_k) + 2048            # beyond the static count table
    l = torch.zeros((1, E), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        # sizes are checked before any pointer is touched: a 1-row logits tensor stands in
        p = moe.RouteParams(E, 8, 4, top_k, 2.827, 1)
        import ctypes
        st = moe.lib.moe_route_permute_noalloc(ctypes.c_void_p(l.data_ptr()), None, T, ctypes.byref(p),
                                               ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                               ctypes.c_void_p(16), ctypes.c_void_p(16), None)
        moe._check(st, "moe_route_permute_noalloc")
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
