"""One routed-expert MoE layer composed from the five C-ABI calls.

route -> permute -> [W4A4: quantise x] -> gate/up grouped GEMM with SwiGLU
(writes z, bf16 or NVFP4) -> down grouped GEMM -> weighted combine.  Buffers
are allocated once for a maximum token count, so a forward pass allocates
nothing and can be captured in a HIP graph.

W4A4: x is quantised to NVFP4 and the gate/up epilogue quantises z to NVFP4;
both GEMMs then multiply the NVFP4 values themselves, handed over as exact
bfloat16 (code x scale x global has at most 6 significant bits), so they run
the bf16-input kernels on exactly the W4A4 operands.  ``a_mode="nvfp4_codes"``
feeds the GEMMs the NVFP4 codes and scales instead (the same products, with
the dequantisation inside the GEMM); ``a_mode="planes"`` feeds them the same
NVFP4 values as two exact E4M3 planes under E8M0 scales, on the block-scaled
MFMA with the FP4 weights as its native operand.

W4A8 (``act_mode="mxfp8"``): x is quantised to MXFP8 and the gate/up epilogue
quantises the bf16 z to MXFP8; both GEMMs run on the block-scaled MFMA.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import (MOE_ALGO_AUTO, Weights, combine, grouped_gemm, permute, permute_workspace_bytes, quantize_mxfp8,
               quantize_nvfp4, quantize_nvfp4_planes, reap_saliency_accumulate, route_gemv, route_gemv_workspace_bytes,
               route_permute)


@dataclasses.dataclass
class LayerWeights:
    gate: Weights     # [E, I, H]
    up: Weights       # [E, I, H]
    down: Weights     # [E, H, I]


class MoELayer:
    def __init__(self, weights: LayerWeights, num_experts: int, n_group: int, topk_group: int, top_k: int,
                 routed_scaling_factor: float, max_tokens: int, act_mode: str = "bf16", input_scale: float = 1.0,
                 keep_z_bf16: bool = False, a_mode: str = "dequant", router_weight: Optional[torch.Tensor] = None,
                 saliency: bool = False, device="cuda"):
        """``router_weight``: FP32 [E, hidden]; with it, forward() may be called
        without logits and runs the router matmul fused with the top-k.
        ``saliency``: every forward also accumulates the REAP saliency of each
        expert (sal_sums / sal_counts; S = sal_sums / sal_counts)."""
        self.w = weights
        self.E, self.n_group, self.topk_group, self.top_k = num_experts, n_group, topk_group, top_k
        self.scale = routed_scaling_factor
        self.act_mode = act_mode
        self.a_mode = a_mode
        self.input_scale = input_scale
        E, I, H2 = weights.gate.packed.shape
        H = 2 * H2
        self.H, self.I = H, I
        T, R = max_tokens, max_tokens * top_k
        dev = torch.device(device)
        i32 = torch.int32
        self.ids = torch.empty((T, top_k), dtype=i32, device=dev)
        self.topw = torch.empty((T, top_k), dtype=torch.float32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.sorted_slots = torch.empty(R, dtype=i32, device=dev)
        self.slot_rows = torch.empty(R, dtype=i32, device=dev)
        self.ws = torch.empty(max(permute_workspace_bytes(T, top_k, E), 16), dtype=torch.uint8, device=dev)
        self.counter = torch.zeros(1, dtype=i32, device=dev)   # router -> permutation hand-off (left zero)
        self.router_weight = router_weight
        self.saliency = saliency
        if saliency:
            self.row_sumsq = torch.empty((R, H // 64), dtype=torch.float32, device=dev)
            self.sal_sums = torch.zeros(E, dtype=torch.float64, device=dev)
            self.sal_counts = torch.zeros(E, dtype=torch.int64, device=dev)
        if router_weight is not None:                           # router matmul: its float64 logits
            self.rws = torch.empty(route_gemv_workspace_bytes(T, E), dtype=torch.uint8, device=dev)
        self.o = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        if act_mode == "mxfp8" or (act_mode == "nvfp4" and a_mode == "planes"):
            planes = act_mode == "nvfp4"
            kx, kz = (2 * H, 2 * I) if planes else (H, I)
            sx, sz = (H // 16, I // 16) if planes else (H // 32, I // 32)
            self.x_q = torch.empty((T, kx), dtype=torch.uint8, device=dev)
            self.x_qs = torch.empty((T, sx), dtype=torch.uint8, device=dev)
            self.z_q = torch.empty((R, kz), dtype=torch.uint8, device=dev)
            self.z_qs = torch.empty((R, sz), dtype=torch.uint8, device=dev)
            self.z = torch.empty((R, I), dtype=torch.bfloat16, device=dev) if keep_z_bf16 else None
            return
        w4a4 = act_mode == "nvfp4"
        self.z = torch.empty((R, I), dtype=torch.bfloat16, device=dev) if (not w4a4 or keep_z_bf16) else None
        if w4a4:
            self.x_codes = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
            self.x_scales = torch.empty((T, H // 16), dtype=torch.uint8, device=dev)
            self.z_codes = torch.empty((R, I // 2), dtype=torch.uint8, device=dev)
            self.z_scales = torch.empty((R, I // 16), dtype=torch.uint8, device=dev)
            if a_mode == "dequant":
                self.x_dq = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
                self.z_dq = torch.empty((R, I), dtype=torch.bfloat16, device=dev)

    def forward(self, x: torch.Tensor, logits: Optional[torch.Tensor], bias: Optional[torch.Tensor] = None,
                residual: Optional[torch.Tensor] = None, algo: int = MOE_ALGO_AUTO, y: Optional[torch.Tensor] = None,
                events: Optional[dict] = None):
        """``events``: optional {step name: (start, end)} torch.cuda.Event pairs recorded
        around the gate/up ("gate_up") and down ("down") GEMM launches."""
        T = x.shape[0]

        def mark(name, i):
            if events is not None and name in events:
                events[name][i].record()
        R = T * self.top_k
        ids, topw = self.ids[:T], self.topw[:T]
        if logits is None:
            # router matmul, its top-k, then the permutation
            route_gemv(x, self.router_weight, bias, self.E, self.n_group, self.topk_group, self.top_k, self.scale,
                       self.rws, True, ids=ids, weights=topw)
            permute(ids, self.E, workspace=self.ws, offsets=self.offsets, sorted_slots=self.sorted_slots[:R],
                    slot_rows=self.slot_rows[:R])
        else:
            route_permute(logits, bias, self.E, self.n_group, self.topk_group, self.top_k, self.scale, self.counter,
                          True, ids=ids, weights=topw, workspace=self.ws, offsets=self.offsets,
                          sorted_slots=self.sorted_slots[:R], slot_rows=self.slot_rows[:R])
        z = None if self.z is None else self.z[:R]
        o = self.o[:R]
        sq = self.row_sumsq[:R] if self.saliency else None
        if self.act_mode == "mxfp8" or (self.act_mode == "nvfp4" and self.a_mode == "planes"):
            planes = self.act_mode == "nvfp4"
            if planes:
                quantize_nvfp4_planes(x, self.input_scale, self.x_q[:T], self.x_qs[:T])
            else:
                quantize_mxfp8(x, self.x_q[:T], self.x_qs[:T])
            am = "planes" if planes else "mxfp8"
            mark("gate_up", 0)
            grouped_gemm(self.x_q[:T], self.w.gate, self.w.up, self.offsets, R, gather=self.sorted_slots[:R],
                         gather_div=self.top_k, a_scales=self.x_qs[:T], out=z, out_codes=self.z_q[:R],
                         out_scales=self.z_qs[:R], output_scale=self.input_scale if planes else 1.0,
                         want_bf16=z is not None, algo=algo, a_mode=am, out_format=am)
            mark("gate_up", 1)
            mark("down", 0)
            grouped_gemm(self.z_q[:R], self.w.down, None, self.offsets, R, a_scales=self.z_qs[:R], out=o, algo=algo,
                         a_mode=am, row_sumsq=sq)
            mark("down", 1)
        elif self.act_mode == "nvfp4" and self.a_mode == "dequant":
            xdq = self.x_dq[:T]
            quantize_nvfp4(x, self.input_scale, self.x_codes[:T], self.x_scales[:T], dequant=xdq)
            keep = z is not None
            mark("gate_up", 0)
            grouped_gemm(xdq, self.w.gate, self.w.up, self.offsets, R, gather=self.sorted_slots[:R],
                         gather_div=self.top_k, out=z, out_codes=self.z_codes[:R] if keep else None,
                         out_scales=self.z_scales[:R] if keep else None, output_scale=self.input_scale,
                         want_bf16=keep, out_dequant=self.z_dq[:R], algo=algo)
            mark("gate_up", 1)
            mark("down", 0)
            grouped_gemm(self.z_dq[:R], self.w.down, None, self.offsets, R, out=o, algo=algo, row_sumsq=sq)
            mark("down", 1)
        elif self.act_mode == "nvfp4":
            xc, xs = quantize_nvfp4(x, self.input_scale, self.x_codes[:T], self.x_scales[:T])
            mark("gate_up", 0)
            grouped_gemm(xc, self.w.gate, self.w.up, self.offsets, R, gather=self.sorted_slots[:R],
                         gather_div=self.top_k, a_scales=xs, input_scale=self.input_scale, out=z,
                         out_codes=self.z_codes[:R], out_scales=self.z_scales[:R], output_scale=self.input_scale,
                         want_bf16=z is not None, algo=algo)
            mark("gate_up", 1)
            mark("down", 0)
            grouped_gemm(self.z_codes[:R], self.w.down, None, self.offsets, R, a_scales=self.z_scales[:R],
                         input_scale=self.input_scale, out=o, algo=algo, row_sumsq=sq)
            mark("down", 1)
        else:
            mark("gate_up", 0)
            grouped_gemm(x, self.w.gate, self.w.up, self.offsets, R, gather=self.sorted_slots[:R],
                         gather_div=self.top_k, out=z, algo=algo)
            mark("gate_up", 1)
            mark("down", 0)
            grouped_gemm(z, self.w.down, None, self.offsets, R, out=o, algo=algo, row_sumsq=sq)
            mark("down", 1)
        if self.saliency:
            reap_saliency_accumulate(sq, self.offsets, self.sorted_slots[:R], topw, self.sal_sums, self.sal_counts, R)
        y = self.y[:T] if y is None else y
        combine(o, self.slot_rows[:R], topw, residual, y=y)
        return y
