"""REAP expert saliency, accumulated over batches (oracle, float64).

[REAP50] "Pruning Method", REAP saliency equation: for every expert j,
S_j = (1 / |T_j|) sum over the tokens t routed to j of g_{t,j} times the L2
norm of expert j's output for token t, W_down,j(SiLU(W_gate,j h_t) (*)
(W_up,j h_t)).

Readings where the page leaves the step open:
  * g_{t,j} is the router weight the layer itself gives expert j's output for
    token t: the normalised top-k weight times routed_scaling_factor, i.e. the
    weight the combine applies;
  * the expert output is the down projection's result before any rounding
    (float64 here);
  * over a calibration stream the numerator and |T_j| are accumulated
    separately, batch by batch, and S_j = numerator / |T_j| (an expert no
    token reached has no saliency).
"""
from __future__ import annotations

import numpy as np


def saliency_accumulate(o: np.ndarray, weights: np.ndarray, ids: np.ndarray, num_experts: int,
                        sums: np.ndarray = None, counts: np.ndarray = None):
    """o float64 [T, top_k, H] expert outputs, weights [T, top_k] (g), ids [T, top_k].
    Adds sum_t g ||o|| and the token counts per expert into (sums f64 [E], counts i64 [E])."""
    sums = np.zeros(num_experts) if sums is None else sums
    counts = np.zeros(num_experts, np.int64) if counts is None else counts
    norms = np.sqrt(np.sum(np.asarray(o, np.float64) ** 2, axis=-1))
    T, k = ids.shape
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            sums[e] += float(weights[t, j]) * norms[t, j]
            counts[e] += 1
    return sums, counts


def saliency(sums: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """S_j = sums_j / counts_j (NaN where no token reached expert j)."""
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(counts > 0, sums / np.maximum(counts, 1), np.nan)
