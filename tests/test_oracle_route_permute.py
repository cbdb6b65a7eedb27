"""Pins for the oracle's routing and permutation (CPU only).

Routing is checked against exhaustive enumeration (every group subset, every
expert subset) and against a straightforward per-token sort written here; the
sigmoid against scipy's expit; the constants against the pages.  The
permutation is checked against per-expert bucket lists built by a loop.
"""
import itertools
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from synth import WORKLOADS, logits as gen_logits, random_logits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _consts():
    d = {}
    with open(os.path.join(GOLD, "routing_constants.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                d[k] = float(v)
    return d


def test_workload_constants_match_pages():
    c = _consts()
    s = WORKLOADS["decode"].shape
    assert (s.num_experts, s.n_group, s.topk_group, s.top_k) == (
        c["n_routed_experts"], c["n_group"], c["topk_group"], c["num_experts_per_tok"])
    assert s.routed_scaling_factor == c["routed_scaling_factor"]
    r = WORKLOADS["reap50"].shape
    assert r.num_experts == c["pruned_experts"] and r.num_experts // r.n_group == c["pruned_experts_per_group"]


def _brute_force_tiny(l, bias, n_group, topk_group, top_k, scale):
    s = expit(l.astype(np.float64))
    c = s + (0 if bias is None else bias.astype(np.float64))
    E = len(l)
    gs = E // n_group
    gscore = [sum(sorted(c[g * gs:(g + 1) * gs])[-2:]) for g in range(n_group)]
    best = max(itertools.combinations(range(n_group), topk_group), key=lambda S: sum(gscore[g] for g in S))
    cand = [e for g in best for e in range(g * gs, (g + 1) * gs)]
    bestE = max(itertools.combinations(cand, top_k), key=lambda S: sum(c[e] for e in S))
    ordered = sorted(bestE, key=lambda e: (-c[e], e))
    w = np.array([s[e] for e in ordered])
    return ordered, w / w.sum() * scale


@pytest.mark.parametrize("with_bias", [False, True])
def test_route_exhaustive_tiny(with_bias):
    w = WORKLOADS["tiny"]
    s = w.shape
    l = gen_logits(w, 32)
    bias = (np.random.default_rng(5).standard_normal(s.num_experts) * 0.5).astype(np.float32) if with_bias else None
    r = oracle.route(l, bias, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
    assert not r.near_tie.any()
    for t in range(l.shape[0]):
        ids, wts = _brute_force_tiny(l[t], bias, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
        assert list(r.ids[t]) == ids
        np.testing.assert_allclose(r.weights[t], wts, rtol=1e-14)
        assert abs(r.weights[t].sum() - 2.827) < 1e-12


def _sort_based(l, bias, n_group, topk_group, top_k, scale):
    out_ids, out_w = [], []
    for row in l:
        s = [1.0 / (1.0 + np.exp(-float(v))) for v in row]
        c = [si + (0.0 if bias is None else float(bias[i])) for i, si in enumerate(s)]
        gs = len(row) // n_group
        gsc = []
        for g in range(n_group):
            top = sorted(c[g * gs:(g + 1) * gs], reverse=True)
            gsc.append((top[0] + top[1], g))
        kept = [g for _, g in sorted(gsc, key=lambda p: (-p[0], p[1]))[:topk_group]]
        cand = sorted([e for g in kept for e in range(g * gs, (g + 1) * gs)], key=lambda e: (-c[e], e))[:top_k]
        ws = np.array([s[e] for e in cand])
        out_ids.append(cand)
        out_w.append(ws / ws.sum() * scale)
    return np.array(out_ids), np.array(out_w)


@pytest.mark.parametrize("name", ["decode", "prefill", "reap50"])
def test_route_matches_sort_based(name):
    w = WORKLOADS[name]
    s = w.shape
    from synth import correction_bias
    l = gen_logits(w, max(w.tokens))[:64]
    bias = correction_bias(w)
    r = oracle.route(l, bias, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
    ids, wts = _sort_based(l, bias, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
    assert np.array_equal(r.ids, ids)
    np.testing.assert_allclose(r.weights, wts, rtol=1e-13)


def test_route_ties_go_to_lower_index():
    l = np.zeros((1, 32), np.float32)      # every score equal
    r = oracle.route(l, None, 8, 4, 8, 2.827)
    # groups 0..3 kept; experts of the first two groups (all equal) in index order
    assert list(r.ids[0]) == list(range(8))
    np.testing.assert_allclose(r.weights[0], np.full(8, 2.827 / 8), rtol=1e-15)


def test_route_bias_only_selects():
    l = random_logits(6, 16, 32)
    bias = np.zeros(32, np.float32)
    bias[31] = 10.0                          # forces expert 31 first, but weight uses sigmoid only
    r = oracle.route(l, bias, 8, 4, 8, 2.827)
    assert np.all(r.ids[:, 0] == 31)
    s = expit(l.astype(np.float64))
    sel = np.take_along_axis(s, r.ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(r.weights, sel / sel.sum(1, keepdims=True) * 2.827, rtol=1e-14)


def test_sigmoid_matches_expit():
    l = random_logits(7, 64, 256)
    r = oracle.route(l, None, 8, 4, 8, 1.0, norm_topk_prob=False)
    sel = np.take_along_axis(expit(l.astype(np.float64)), r.ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(r.weights, sel, rtol=1e-15)


def test_permute_against_buckets():
    rng = np.random.default_rng(8)
    for T, E in [(0, 8), (1, 256), (37, 32), (513, 256), (300, 128)]:
        ids = rng.integers(0, E, size=(T, 8)).astype(np.int32)
        off, ss, sr = oracle.permute(ids, E)
        buckets = [[] for _ in range(E)]
        for slot, e in enumerate(ids.ravel()):
            buckets[e].append(slot)
        flat = [s for b in buckets for s in b]
        assert list(ss) == flat
        assert list(off) == list(np.cumsum([0] + [len(b) for b in buckets]))
        assert off[-1] == T * 8
        for row, slot in enumerate(ss):
            assert sr[slot] == row


def _tie_case(gap_expert: float, gap_group: float):
    """One token whose every routing decision is fixed by construction (all
    biases are powers of two or small dyadic values, exact in float32):
    experts with logit 0 have sigmoid exactly 1/2, the others logit -4.
    Seven experts lead clearly (0, 1, 8, 9, 16, 17, 24); the 8th place goes to
    expert 2 (1/2 + gap_expert) over expert 3 (1/2); group 3 beats group 4 for
    the 4th kept group by gap_group (its second expert carries the gap)."""
    E = 64
    l = np.full((1, E), -4.0, np.float32)
    b = np.zeros(E, np.float64)
    for e, bias in ((0, 0.375), (1, 0.375), (8, 0.25), (9, 0.25), (16, 0.125), (17, 0.125), (24, 0.125),
                    (32, 0.125), (2, gap_expert), (3, 0.0)):
        l[0, e] = 0.0
        b[e] = bias
    b[25] = gap_group            # logit -4: group 3 = 0.625 + (s + gap), group 4 = 0.625 + s
    return l, b.astype(np.float32)


@pytest.mark.parametrize("gap_expert,gap_group,flag", [
    (2.0 ** -41, 2.0 ** -4, True),      # 8th/9th expert gap 4.5e-13 < 1e-12
    (2.0 ** -38, 2.0 ** -4, False),     # 3.6e-12: a clear decision
    (2.0 ** -4, 2.0 ** -42, True),      # 4th/5th group gap 2.3e-13
    (2.0 ** -4, 2.0 ** -36, False),     # 1.5e-11
    (0.0, 2.0 ** -4, False),            # an exact tie is decided by index, not flagged
])
def test_near_tie_flag_on_constructed_gaps(gap_expert, gap_group, flag):
    """near_tie marks exactly the tokens whose 8th/9th expert or 4th/5th group
    decision has a gap in (0, 1e-12); the decisions themselves go the way the
    constructed gaps (or, at an exact tie, the lower index) say."""
    l, b = _tie_case(gap_expert, gap_group)
    assert np.array_equal(b.astype(np.float64)[[2, 25]], [gap_expert, gap_group])   # exact in float32
    r = oracle.route(l, b, 8, 4, 8, 2.827)
    assert bool(r.near_tie[0]) == flag
    assert sorted(r.ids[0][:7].tolist()) == [0, 1, 8, 9, 16, 17, 24]
    assert r.ids[0][7] == 2
    assert sorted({int(e) // 8 for e in r.ids[0]}) == [0, 1, 2, 3]


# ------------------------------------------------ router matmul + top-k
def test_router_logits_within_float64_sum_bound():
    """The float64 router matmul against exact rational dot products: every
    product bf16 x FP32 is exact, so the only error is the float64 summation,
    bounded by (H - 1) 2^-53 sum_k |x_k W_ek|."""
    from fractions import Fraction
    from synth import router_weight
    w = WORKLOADS["decode"]
    W = router_weight(w)[:6]
    x = random_bf16_bits(7, (3, W.shape[1]))
    l = oracle.router_logits(x, W)
    xv = oracle.bf16_value(x)
    H = W.shape[1]
    for t in range(3):
        for e in range(6):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[t], W[e].astype(np.float64)))
            bound = (H - 1) * 2.0 ** -53 * float(np.sum(np.abs(xv[t] * W[e].astype(np.float64))))
            assert abs(Fraction(l[t, e]) - exact) <= Fraction(bound)


def test_route_hidden_exhaustive_tiny():
    """Routing from the float64 router logits agrees with exhaustive enumeration
    of the group and expert subsets (the brute force of the FP32-logit pin, fed
    the same float64 logits)."""
    from synth import router_weight
    w = WORKLOADS["tiny"]
    s = w.shape
    x = random_bf16_bits(8, (16, s.hidden))
    W = router_weight(w)
    r, l = oracle.route_hidden(x, W, None, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
    for t in range(16):
        ids, wts = _brute_force_tiny(l[t], None, s.n_group, s.topk_group, s.top_k, s.routed_scaling_factor)
        assert list(r.ids[t]) == ids
        np.testing.assert_allclose(r.weights[t], wts, rtol=1e-12)


def random_bf16_bits(seed, shape):
    from synth import random_bf16
    return random_bf16(seed, shape)
