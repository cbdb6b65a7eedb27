"""Group-limited sigmoid top-k routing (oracle, float64).

[REAP50] "Pruning Method", group-balanced REAP saliency paragraph: MiMo uses
grouped sigmoid top-k routing with n_routed_experts = 256 in n_group = 8
groups, topk_group = 4, num_experts_per_tok = 8, routed_scaling_factor = 2.827,
and the router reshapes experts into [n_group, n_routed_experts // n_group].
[REAP50] "Evaluation Status Note": the router carries ``e_score_correction_bias``.
[GGUF] "Quantization targets": routers are kept in F32.

Readings where the pages are silent:
  * score s_e = sigmoid(logit_e) in float64; the correction bias is added for
    selection only, c_e = s_e + bias_e; the returned weights use s_e;
  * group score = sum of the two largest c_e in the group (``group_score="max"``
    switches to the largest one);
  * keep the topk_group groups with the largest group score, then take the
    top_k largest c_e among experts of kept groups (others are excluded);
  * ties go to the lower group / expert index; ids are listed by c descending;
  * weights: w_j = s_{e_j} / sum_j s_{e_j} * routed_scaling_factor (with
    ``norm_topk_prob``), else s_{e_j} * routed_scaling_factor.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

NEAR_TIE = 1e-12


@dataclasses.dataclass
class RouteResult:
    ids: np.ndarray        # int32 [T, top_k]
    weights: np.ndarray    # float64 [T, top_k]
    near_tie: np.ndarray   # bool [T]: a decision gap in (0, 1e-12)


def _order_desc(values: np.ndarray) -> np.ndarray:
    """Per row, indices sorted by value descending, ties by index ascending."""
    idx = np.broadcast_to(np.arange(values.shape[-1]), values.shape)
    return np.lexsort((idx, -values), axis=-1)


def route(logits: np.ndarray, bias: Optional[np.ndarray], n_group: int, topk_group: int,
          top_k: int, routed_scaling_factor: float, norm_topk_prob: bool = True,
          group_score: str = "top2") -> RouteResult:
    """Routing from FP32 logits (the router's output as stored)."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    return route_f64(l, bias, n_group, topk_group, top_k, routed_scaling_factor, norm_topk_prob, group_score)


def router_logits(x_bits: np.ndarray, gate_weight: np.ndarray) -> np.ndarray:
    """The router's matmul in float64: logits[t, e] = sum_k x[t, k] W[e, k] for
    bf16 hidden states x and the FP32 router weight W [E, H] ([GGUF]
    "Quantization targets": routers stay F32).  Every product of a bf16 and an
    FP32 value is exact in float64; only the sum rounds."""
    from .formats import bf16_value
    return bf16_value(x_bits) @ np.asarray(gate_weight, np.float32).astype(np.float64).T


def route_hidden(x_bits: np.ndarray, gate_weight: np.ndarray, bias: Optional[np.ndarray], n_group: int,
                 topk_group: int, top_k: int, routed_scaling_factor: float, norm_topk_prob: bool = True):
    """[PRO6000] "What makes it fast": the router's matmul and the top-k in one
    step.  Reading: the float64 logits of router_logits feed the selection
    directly (no rounding to FP32 in between).  Returns (RouteResult, logits)."""
    l = router_logits(x_bits, gate_weight)
    return route_f64(l, bias, n_group, topk_group, top_k, routed_scaling_factor, norm_topk_prob), l


def route_f64(l: np.ndarray, bias: Optional[np.ndarray], n_group: int, topk_group: int,
              top_k: int, routed_scaling_factor: float, norm_topk_prob: bool = True,
              group_score: str = "top2") -> RouteResult:
    """Routing from float64 logits l [T, E] (the steps of the module docstring)."""
    T, E = l.shape
    gs = E // n_group
    s = 1.0 / (1.0 + np.exp(-l))
    c = s + (0.0 if bias is None else np.asarray(bias, np.float32).astype(np.float64)[None, :])

    grouped = c.reshape(T, n_group, gs)
    desc = -np.sort(-grouped, axis=-1)
    if group_score == "top2":
        g = desc[..., 0] + desc[..., 1]
    elif group_score == "max":
        g = desc[..., 0]
    else:
        raise ValueError(group_score)

    gorder = _order_desc(g)
    kept = gorder[:, :topk_group]
    keep_mask = np.zeros((T, n_group), bool)
    np.put_along_axis(keep_mask, kept, True, axis=1)
    expert_keep = np.repeat(keep_mask, gs, axis=1)
    cand = np.where(expert_keep, c, -np.inf)

    eorder = _order_desc(cand)
    ids = eorder[:, :top_k]

    sel_s = np.take_along_axis(s, ids, axis=1)
    if norm_topk_prob:
        w = sel_s / sel_s.sum(axis=1, keepdims=True) * routed_scaling_factor
    else:
        w = sel_s * routed_scaling_factor

    gsorted = np.take_along_axis(g, gorder, axis=1)
    csorted = np.take_along_axis(cand, eorder, axis=1)
    near = np.zeros(T, bool)
    if topk_group < n_group:
        d = gsorted[:, topk_group - 1] - gsorted[:, topk_group]
        near |= (d > 0) & (d < NEAR_TIE)
    if top_k < topk_group * gs:
        d = csorted[:, top_k - 1] - csorted[:, top_k]
        near |= (d > 0) & (d < NEAR_TIE)
    return RouteResult(ids=ids.astype(np.int32), weights=w, near_tie=near)
