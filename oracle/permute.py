"""Token permutation: group the (token, k) slots by expert (oracle).

[PRO6000] "What makes it fast", speed-v4 list: short prompts run through one
grouped kernel over the routed experts; grouping requires each expert's rows to
be contiguous.  The pages do not describe the permutation itself.

Reading adopted: slot s = t * top_k + j; a stable sort of slots by expert id
(ascending slot order inside an expert); ``expert_offsets`` is the exclusive
prefix sum of per-expert counts (length E+1); ``slot_rows`` is the inverse
permutation (slot -> permuted row).
"""
from __future__ import annotations

import numpy as np


def permute(ids: np.ndarray, num_experts: int):
    flat = np.asarray(ids, dtype=np.int64).ravel()
    sorted_slots = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    slot_rows = np.empty_like(sorted_slots)
    slot_rows[sorted_slots] = np.arange(flat.size)
    return offsets.astype(np.int32), sorted_slots.astype(np.int32), slot_rows.astype(np.int32)
