"""CPU oracle for the FP4 routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy statement of what the layer computes, written from
the pages (cited per function).  It shares no code with the HIP path and is used
only by ``tests/``, the smoke check and the CPU-baseline leg of ``bench.py``;
the product path never calls it and never falls back to it.

Citations name the page and its section:
  [MOPD-NVFP4]  "AxionML / MiMo-V2.6-Flash-MOPD-NVFP4" model card
  [RL-NVFP4]    "MiMo-V2.6-Flash-RL: exact NVFP4 weight conversion" card
  [GGUF]        "MiMo-V2.6-Flash-RL Mixed-Quant GGUF" card
  [REAP50]      "MiMo-V2.6-Flash -- REAP-50 (MXFP4 + FP8 Master Checkpoint)" card
  [PRO6000]     "MiMo-V2.6-Flash-MOPD on one RTX PRO 6000" recipe

Every function is pinned by a CPU test against something other than itself
(library codecs, brute force, closed forms, the pages' printed values).  One
convention has no such pin and is marked "parity unpinned" where it is
defined: the choice of the transcode's global scale exponent (many choices are
exact; the pages do not say which one they used).
"""
from .formats import (E2M1_MAGNITUDES, e2m1_value, e8m0_value, e4m3_value, round_to_e4m3,
                      round_to_e2m1_magnitude, bf16_value, round_to_bf16_bits,
                      unpack_codes, dequant_mx, dequant_nv)
from .transcode import transcode_mx_to_nv
from .route import route, route_f64, route_hidden, router_logits, RouteResult
from .permute import permute
from .quant import quantize_nvfp4, dequant_nvfp4_act, quantize_mxfp8, dequant_mxfp8
from .layer import silu, expert_ffn, combine, combine_f64, moe_layer, LayerResult
from .saliency import saliency_accumulate, saliency
from .compact import compact_mx, dequant_compact

__all__ = [
    "E2M1_MAGNITUDES", "e2m1_value", "e8m0_value", "e4m3_value", "round_to_e4m3",
    "round_to_e2m1_magnitude", "bf16_value", "round_to_bf16_bits", "unpack_codes",
    "dequant_mx", "dequant_nv", "transcode_mx_to_nv", "route", "route_f64", "route_hidden", "router_logits", "RouteResult", "permute",
    "quantize_nvfp4", "dequant_nvfp4_act", "quantize_mxfp8", "dequant_mxfp8", "silu", "expert_ffn", "combine", "combine_f64", "moe_layer",
    "LayerResult", "saliency_accumulate", "saliency", "compact_mx", "dequant_compact",
]
