"""Seeded synthetic inputs for the FP4 routed-expert MoE layer.

This module draws random numbers and lays them out in the storage formats the
layer consumes; it holds none of the layer's arithmetic (no decoding, routing,
quantisation or matrix products).  Both the CPU oracle and the HIP path are fed
from here, so they always see identical bytes.

Shapes follow the pages:
  * 256 routed experts in 8 groups, keep 4 groups, 8 experts per token, scaling
    2.827 (MiMo-V2.6-Flash-REAP50 card, "Pruning Method", group-balanced REAP
    saliency paragraph; model-summary table); 128 experts in 8 groups of 16 for
    the REAP-50 shape (same card, model-summary table).
  * each routed-expert matrix holds 4096 x 2048 values: the exact-NVFP4 card's
    "Verification" table counts 302,795,194,368 expert values, i.e. 47 MoE
    layers x 256 experts x 3 matrices x 8,388,608 values.
  * MXFP4 expert storage: E2M1 codes packed two per byte ("weight_packed" U8)
    with one E8M0 scale per 32 values ("weight_scale"), REAP50 card,
    "Highlights".
  * activation outliers of amax 2,960 / 18,560 / 311,296 at the down-projection
    input (MOPD-NVFP4 card, "Quantization Details").

Recipe (every tensor): numpy ``default_rng(SeedSequence([2026, workload id,
layer, tensor id, tokens]))``; tensor ids: 0 logits, 1 correction bias, 2 x,
3/4 gate codes/exponents, 5/6 up, 7/8 down, 9 synthetic down-proj input,
10 outlier positions, 11 Zipf expert ranks, 12 router weight.
  * codes: uniform random bytes (both nibbles uniform over all 16 E2M1 codes,
    including -0);
  * E8M0 scale bytes: uniform in {119..125}, i.e. 2^-8 .. 2^-2;
  * router logits: float32 N(0,1); REAP-50 shape adds ln p_r(e) with
    p_r proportional to r^-1.1 over a seeded rank permutation r(e);
  * correction bias: float32 N(0, 0.5) for the prefill shape, absent elsewhere;
  * router weight (the FP32 gate.weight [E, hidden] for the fused router):
    float32 N(0, 1/hidden), so that its logits on N(0,1) activations are
    about N(0,1), like the synthetic logits;
  * activations: N(0,1) rounded to bfloat16 (round-to-nearest-even, done by
    torch's dtype conversion).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_ROOT = 2026

T_LOGITS, T_BIAS, T_X = 0, 1, 2
T_GATE_CODES, T_GATE_EXP, T_UP_CODES, T_UP_EXP, T_DOWN_CODES, T_DOWN_EXP = 3, 4, 5, 6, 7, 8
T_ZSYN, T_OUTLIER_POS, T_ZIPF = 9, 10, 11
T_ROUTER_W = 12

E8M0_LO, E8M0_HI = 119, 125          # inclusive: 2^-8 .. 2^-2
OUTLIER_AMAX = (2960.0, 18560.0, 311296.0)
OUTLIER_FRACTION = 1e-3


@dataclasses.dataclass(frozen=True)
class LayerShape:
    num_experts: int
    n_group: int
    topk_group: int
    top_k: int
    hidden: int
    inter: int
    routed_scaling_factor: float = 2.827


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    shape: LayerShape
    tokens: tuple
    layers: int = 1
    bias_std: float = 0.0
    zipf_s: float = 0.0
    act_mode: str = "bf16"       # "bf16" (W4A16) or "nvfp4" (W4A4)
    weight_format: str = "mx"    # "mx" or "nv" (exact transcode of the MX weights)
    weight_wid: Optional[int] = None  # draw weights with another workload's seeds


FULL = LayerShape(num_experts=256, n_group=8, topk_group=4, top_k=8, hidden=4096, inter=2048)
REAP = LayerShape(num_experts=128, n_group=8, topk_group=4, top_k=8, hidden=4096, inter=2048)
TINY = LayerShape(num_experts=32, n_group=8, topk_group=4, top_k=8, hidden=512, inter=256)

WORKLOADS = {
    "tiny": Workload("tiny", 1, TINY, (32,)),
    "decode": Workload("decode", 2, FULL, (1, 8, 64)),
    "prefill": Workload("prefill", 3, FULL, (8192,), bias_std=0.5),
    "w4a4": Workload("w4a4", 4, FULL, (4096,), act_mode="nvfp4", weight_format="nv", weight_wid=2),
    "reap50": Workload("reap50", 5, REAP, (16384,), layers=2, zipf_s=1.1),
}


def rng(wid: int, layer: int, tensor: int, tokens: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, wid, layer, tensor, tokens]))


def random_bytes(g: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    words = g.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n].reshape(shape).copy()


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16) via torch's own conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def logits(w: Workload, T: int, layer: int = 0) -> np.ndarray:
    E = w.shape.num_experts
    g = rng(w.wid, layer, T_LOGITS, T)
    out = g.standard_normal((T, E), dtype=np.float64)
    if w.zipf_s:
        perm = rng(w.wid, layer, T_ZIPF).permutation(E) + 1          # rank of each expert, 1..E
        p = perm.astype(np.float64) ** (-w.zipf_s)
        p /= p.sum()
        out = out + np.log(p)[None, :]
    return out.astype(np.float32)


def router_weight(w: Workload, layer: int = 0) -> np.ndarray:
    """FP32 router weight [E, hidden], N(0, 1/hidden)."""
    g = rng(w.wid, layer, T_ROUTER_W)
    H = w.shape.hidden
    return (g.standard_normal((w.shape.num_experts, H)) / np.sqrt(H)).astype(np.float32)


def correction_bias(w: Workload, layer: int = 0) -> Optional[np.ndarray]:
    if not w.bias_std:
        return None
    g = rng(w.wid, layer, T_BIAS)
    return (g.standard_normal(w.shape.num_experts) * w.bias_std).astype(np.float32)


def activations(w: Workload, T: int, layer: int = 0) -> np.ndarray:
    """bf16 bit patterns [T, hidden]."""
    g = rng(w.wid, layer, T_X, T)
    return bf16_bits_from_f32(g.standard_normal((T, w.shape.hidden), dtype=np.float32))


def mx_matrix(wid: int, layer: int, codes_id: int, exp_id: int, E: int, n: int, k: int,
              experts: Optional[np.ndarray] = None):
    """MXFP4 weights for E experts of an [n, k] matrix: (packed u8 [E,n,k/2], e8m0 u8 [E,n,k/32]).

    With ``experts`` given, only those experts are drawn (each expert has its own
    stream, so a subset matches the corresponding slices of the full draw).
    """
    idx = range(E) if experts is None else [int(e) for e in experts]
    packed = np.empty((len(idx), n, k // 2), np.uint8)
    scale = np.empty((len(idx), n, k // 32), np.uint8)
    for i, e in enumerate(idx):
        packed[i] = random_bytes(rng(wid, layer, codes_id, e), (n, k // 2))
        scale[i] = rng(wid, layer, exp_id, e).integers(E8M0_LO, E8M0_HI + 1, size=(n, k // 32), dtype=np.uint8)
    return packed, scale


def expert_weights(w: Workload, layer: int = 0, experts: Optional[np.ndarray] = None) -> dict:
    """MXFP4 gate/up/down weights in nn.Linear [out, in] layout per expert."""
    s = w.shape
    wid = w.weight_wid if w.weight_wid is not None else w.wid
    E = s.num_experts
    gate = mx_matrix(wid, layer, T_GATE_CODES, T_GATE_EXP, E, s.inter, s.hidden, experts)
    up = mx_matrix(wid, layer, T_UP_CODES, T_UP_EXP, E, s.inter, s.hidden, experts)
    down = mx_matrix(wid, layer, T_DOWN_CODES, T_DOWN_EXP, E, s.hidden, s.inter, experts)
    return {"gate": gate, "up": up, "down": down}


def down_inputs_with_outliers(rows: int, cols: int, amax: float, seed_layer: int = 0):
    """Synthetic down-projection input: bf16 N(0,1) with a seeded 0.1% of
    positions set to +-amax (all three amax values are exact in bfloat16)."""
    g = rng(4, seed_layer, T_ZSYN, rows)
    z = g.standard_normal((rows, cols), dtype=np.float32)
    gp = rng(4, seed_layer, T_OUTLIER_POS, rows)
    n_out = int(round(rows * cols * OUTLIER_FRACTION))
    pos = gp.choice(rows * cols, size=n_out, replace=False)
    sign = np.where(gp.integers(0, 2, size=n_out) == 1, 1.0, -1.0).astype(np.float32)
    flat = z.reshape(-1)
    flat[pos] = sign * np.float32(amax)
    return bf16_bits_from_f32(z)


def random_mx_small(seed: int, E: int, n: int, k: int, lo: int = E8M0_LO, hi: int = E8M0_HI):
    """Small ad-hoc MXFP4 weights for tests (ragged shapes, edge cases)."""
    g = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 99, seed]))
    packed = random_bytes(g, (E, n, k // 2))
    scale = g.integers(lo, hi + 1, size=(E, n, k // 32), dtype=np.uint8)
    return packed, scale


def random_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 98, seed]))
    return bf16_bits_from_f32((g.standard_normal(shape) * std).astype(np.float32))


def random_logits(seed: int, T: int, E: int) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 97, seed]))
    return g.standard_normal((T, E), dtype=np.float32)
