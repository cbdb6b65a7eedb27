"""Routed-expert MoE layer end to end (oracle, float64).

[REAP50] "Pruning Method", REAP saliency equation: expert j's output for token
t is W_down,j( SiLU(W_gate,j h_t) (elementwise *) (W_up,j h_t) ), weighted by the
router's g_{t,j}.  [MOPD-NVFP4] header paragraph: FP32 (here float64)
accumulation; "Usage" (BF16-activation mode) and "Accuracy": W4A16 (bfloat16
activations) and W4A4 (NVFP4 activations, unit global scale) variants.
[PRO6000] "Quantization, context and quality", Activations: the W4A8 variant
with MXFP8 activations (E4M3, power-of-two scale per 32) for both expert GEMMs.

Roundings happen only where the method stores a narrower type: the layer input
and output are bfloat16, the expert intermediate z = SiLU(gate) * up is stored
as bfloat16 and, in W4A4 / W4A8, re-quantised to NVFP4 / MXFP8 before the
down projection;
everything else is float64.  The combine adds the optional residual and the
router-weighted expert outputs in slot order j = 0..top_k-1.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Sequence

import numpy as np

from .formats import bf16_value, dequant_mx, dequant_nv, round_to_bf16_bits
from .permute import permute
from .quant import dequant_mxfp8, dequant_nvfp4_act, quantize_mxfp8, quantize_nvfp4
from .route import route


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def _act_values(bits: np.ndarray, act_mode: str, input_scale: float) -> np.ndarray:
    if act_mode == "bf16":
        return bf16_value(bits)
    if act_mode == "nvfp4":
        codes, scales = quantize_nvfp4(bits, input_scale)
        return dequant_nvfp4_act(codes, scales, input_scale)
    if act_mode == "mxfp8":
        return dequant_mxfp8(*quantize_mxfp8(bits))
    raise ValueError(act_mode)


def expert_ffn(x_bits: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: Optional[np.ndarray],
               act_mode: str = "bf16", input_scale: float = 1.0):
    """One expert on rows x (bf16 bits [m, H]); weights float64 [I,H], [I,H], [H,I].
    Returns (z bf16 bits [m, I], o float64 [m, H] or None)."""
    a = _act_values(x_bits, act_mode, input_scale)
    gate = a @ wg.T
    up = a @ wu.T
    z_bits = round_to_bf16_bits(silu(gate) * up)
    if wd is None:
        return z_bits, None
    o = _act_values(z_bits, act_mode, input_scale) @ wd.T
    return z_bits, o


def down_proj(z_bits: np.ndarray, wd: np.ndarray, act_mode: str = "bf16", input_scale: float = 1.0):
    return _act_values(z_bits, act_mode, input_scale) @ wd.T


def combine_f64(o: np.ndarray, weights: np.ndarray, residual_bits: Optional[np.ndarray] = None) -> np.ndarray:
    """o float64 [T, top_k, H], weights [T, top_k] -> the layer output in
    float64 [T, H], before its one rounding to bfloat16."""
    acc = np.zeros((o.shape[0], o.shape[2])) if residual_bits is None else bf16_value(residual_bits).copy()
    for j in range(o.shape[1]):
        acc = acc + weights[:, j:j + 1] * o[:, j, :]
    return acc


def combine(o: np.ndarray, weights: np.ndarray, residual_bits: Optional[np.ndarray] = None) -> np.ndarray:
    """o float64 [T, top_k, H], weights [T, top_k] -> y bf16 bits [T, H]."""
    return round_to_bf16_bits(combine_f64(o, weights, residual_bits))


def dequant_expert(weights: dict, e: int, fmt: str):
    """weights: {"gate"|"up"|"down": (packed, scale[, global])} with an expert axis."""
    out = []
    for name in ("gate", "up", "down"):
        t = weights[name]
        if fmt == "mx":
            out.append(dequant_mx(t[0][e], t[1][e]))
        else:
            out.append(dequant_nv(t[0][e], t[1][e], t[2][e]))
    return out


@dataclasses.dataclass
class LayerResult:
    ids: np.ndarray
    weights: np.ndarray
    near_tie: np.ndarray
    offsets: np.ndarray
    sorted_slots: np.ndarray
    slot_rows: np.ndarray
    tokens: np.ndarray               # which tokens z/o/y cover
    z: np.ndarray                    # bf16 bits [len(tokens), top_k, I]
    o: np.ndarray                    # float64 [len(tokens), top_k, H]
    y: np.ndarray                    # bf16 bits [len(tokens), H]
    y_f64: np.ndarray                # float64 [len(tokens), H]: y before its bf16 rounding


def moe_layer(x_bits: np.ndarray, logits: np.ndarray, bias: Optional[np.ndarray], weights: dict,
              n_group: int, topk_group: int, top_k: int, routed_scaling_factor: float,
              fmt: str = "mx", act_mode: str = "bf16", input_scale: float = 1.0,
              residual_bits: Optional[np.ndarray] = None, tokens: Optional[Sequence[int]] = None,
              expert_loader: Optional[Callable[[int], list]] = None) -> LayerResult:
    """The whole layer.  Routing and permutation cover every token; the expert
    FFN and combine are evaluated for ``tokens`` (all by default), one expert at
    a time.  ``expert_loader(e)`` may supply float64 (gate, up, down) for
    expert e instead of dequantising from ``weights``."""
    T, E = logits.shape
    r = route(logits, bias, n_group, topk_group, top_k, routed_scaling_factor)
    offsets, sorted_slots, slot_rows = permute(r.ids, E)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    H = x_bits.shape[1]
    sub_ids = r.ids[toks]
    z = None
    o = np.zeros((len(toks), top_k, H))
    for e in np.unique(sub_ids):
        where = np.argwhere(sub_ids == e)          # (token position, j)
        if expert_loader is not None:
            wg, wu, wd = expert_loader(int(e))
        else:
            wg, wu, wd = dequant_expert(weights, int(e), fmt)
        ze, oe = expert_ffn(x_bits[toks[where[:, 0]]], wg, wu, wd, act_mode, input_scale)
        if z is None:
            z = np.zeros((len(toks), top_k, ze.shape[1]), np.uint16)
        z[where[:, 0], where[:, 1]] = ze
        o[where[:, 0], where[:, 1]] = oe
    res = None if residual_bits is None else residual_bits[toks]
    y_f64 = combine_f64(o, r.weights[toks], res)
    return LayerResult(ids=r.ids, weights=r.weights, near_tie=r.near_tie, offsets=offsets,
                       sorted_slots=sorted_slots, slot_rows=slot_rows, tokens=toks, z=z, o=o,
                       y=round_to_bf16_bits(y_f64), y_f64=y_f64)
