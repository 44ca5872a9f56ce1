"""Pins of the oracle's router against values fixed outside it.

* hand cases with exact dyadic values (tests/golden/hand_cases.json);
* brute-force enumeration with exact rationals (oracle/brute.py is an
  independent formulation: subset enumeration, not sorting);
* invariants the pages fix (K experts, at most M groups, gates from the
  unbiased s summing to 1, load conservation, bias step signs);
* sigmoid against mpmath at 50 digits; logits against exact rational dot
  products.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute, routing

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _cases():
    with open(GOLD) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _cases()["cases"], ids=lambda c: c["name"])
def test_hand_cases(case):
    s = np.array(case["s"], dtype=np.float32)
    b = np.array(case["b"], dtype=np.float32)
    r = routing.select(s, b, case["top_k"], case["n_groups"], case["topk_groups"],
                       case["group_topk"], case.get("group_score_biased", 1))
    assert r.idx.tolist() == case["idx"]
    for t in range(s.shape[0]):
        for k in range(case["top_k"]):
            exact = Fraction(case["gate_num"][t][k], case["gate_den"][k])
            assert abs(Fraction(float(r.gate[t, k])) - exact) <= Fraction(1, 2 ** 52)
    if "keys" in case:
        assert r.key.tolist() == case["keys"]
    if "group_scores" in case:
        assert r.gscore.tolist() == case["group_scores"]
        assert sorted(r.groups[0].tolist()) == sorted(case["groups"][0])
    if "ungrouped_idx" in case:
        r2 = routing.select(s, b, case["top_k"])
        assert r2.idx.tolist() == case["ungrouped_idx"]
    # the brute-force enumerator agrees as a set
    ex, gr = brute.select_one(s[0], b, case["top_k"], case["n_groups"], case["topk_groups"],
                              case["group_topk"], case.get("group_score_biased", 1))
    assert sorted(ex) == sorted(case["idx"][0])


def test_bias_hand_case_c4():
    c = _cases()["bias_cases"][0]
    idx = np.array(c["idx"])
    counts = np.bincount(idx.reshape(-1), minlength=c["n_routed"])
    assert counts.tolist() == c["counts"]
    assert counts.sum() == c["T"] * c["top_k"]
    b0 = np.zeros(c["n_routed"], dtype=np.float32)
    b1 = routing.bias_step(counts, b0, c["T"], c["top_k"], 0.001)
    g = np.float32(0.001)
    assert b1.tolist() == [float(np.float32(d) * g) if d else 0.0 for d in c["delta"]]


def test_bias_forced_routing_c5():
    # b_i = +10 for the first K experts forces every token onto them (s in (0,1))
    rng = np.random.default_rng(5)
    T, N, K = 32, 16, 4
    s = rng.uniform(0.01, 0.99, (T, N)).astype(np.float32)
    b = np.zeros(N, dtype=np.float32)
    b[:K] = 10.0
    r = routing.select(s, b, K)
    assert (np.sort(r.idx, axis=1) == np.arange(K)).all()
    assert r.counts.tolist() == [T] * K + [0] * (N - K)
    b1 = routing.bias_step(r.counts, b, T, K)
    g = np.float32(0.001)
    assert b1[:K].tolist() == [float(np.float32(np.float32(10.0) - g))] * K
    assert b1[K:].tolist() == [float(g)] * (N - K)
    # grouped, biased group scores: group 0 (experts 0..3) carries the forced experts
    r2 = routing.select(s, b, K, n_groups=4, topk_groups=2, group_topk=2)
    assert (np.sort(r2.idx, axis=1) == np.arange(K)).all()


def test_bias_step_values_from_zero():
    rng = np.random.default_rng(1)
    T, N, K = 200, 32, 4
    counts = np.bincount(rng.integers(0, N, T * K), minlength=N)
    b = routing.bias_step(counts, np.zeros(N, np.float32), T, K)
    g = np.float32(0.001)
    mean = T * K / N
    for c, bi in zip(counts, b):
        want = -g if c > mean else (g if c < mean else 0.0)
        assert bi == np.float32(want)


def _random_s(rng, T, N, tie_heavy):
    if tie_heavy:
        # few distinct dyadic values: many exact ties in keys and group sums
        return rng.choice(np.array([0.125, 0.25, 0.375, 0.5, 0.625, 0.75], np.float32), (T, N))
    return rng.uniform(0, 1, (T, N)).astype(np.float32)


SHAPES = [  # N, K, G, M, q
    (8, 4, 4, 2, 2),
    (16, 4, 4, 2, 2),
    (6, 3, 1, 1, None),
    (12, 2, 3, 2, 1),
    (12, 6, 6, 3, 2),
    (16, 8, 8, 4, 2),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "N%d_K%d_G%d_M%d" % s[:4])
@pytest.mark.parametrize("tie_heavy", [False, True])
@pytest.mark.parametrize("biased", [1, 0])
def test_brute_force_matches(shape, tie_heavy, biased):
    N, K, G, M, q = shape
    rng = np.random.default_rng(hash((shape, tie_heavy, biased)) % 2 ** 32)
    for trial in range(6):
        T = 8
        s = _random_s(rng, T, N, tie_heavy)
        b = (rng.choice(np.array([0, 0.125, -0.125, 0.25], np.float32), N) if tie_heavy
             else rng.uniform(-0.05, 0.05, N).astype(np.float32))
        r = routing.select(s, b, K, G, M, q, biased)
        for t in range(T):
            ex, gr = brute.select_one(s[t], b, K, G, M, q, biased)
            assert tuple(sorted(r.idx[t].tolist())) == ex, (t, s[t], b)
            if G > 1:
                assert tuple(sorted(r.groups[t].tolist())) == gr


def test_invariants_v3_shape():
    rng = np.random.default_rng(3)
    T, N, K, G, M, q = 512, 256, 8, 8, 4, 2
    s = rng.uniform(0, 1, (T, N)).astype(np.float32)
    b = rng.uniform(-0.01, 0.01, N).astype(np.float32)
    r = routing.select(s, b, K, G, M, q)
    size = N // G
    keys = routing.keys(s, b)
    for t in range(T):
        sel = r.idx[t]
        assert len(set(sel.tolist())) == K
        grp = set((sel // size).tolist())
        assert len(grp) <= M and grp <= set(r.groups[t].tolist())
        # no candidate outside the selection beats the weakest selected key
        cand = np.nonzero(r.cand[t])[0]
        rest = np.setdiff1d(cand, sel)
        assert keys[t, rest].max() <= keys[t, sel].min()
        # keys in rank order, ties by index
        ks = keys[t, sel]
        assert all(ks[i] > ks[i + 1] or (ks[i] == ks[i + 1] and sel[i] < sel[i + 1]) for i in range(K - 1))
        # chosen groups score at least as high as the others
        gs = r.gscore[t]
        other = np.setdiff1d(np.arange(G), r.groups[t])
        assert gs[r.groups[t]].min() >= gs[other].max()
    # gates: sum to 1, proportional to the unbiased s
    assert np.allclose(r.gate.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    ssel = np.take_along_axis(s.astype(np.float64), r.idx, axis=1)
    assert np.allclose(r.gate * ssel.sum(axis=1, keepdims=True), ssel, rtol=1e-15, atol=0)
    assert r.counts.sum() == T * K
    assert (np.bincount(r.idx.reshape(-1), minlength=N) == r.counts).all()


def test_gate_zero_sum_gives_uniform():
    s = np.zeros((1, 4), np.float32)
    r = routing.select(s, np.zeros(4, np.float32), 2)
    assert r.idx.tolist() == [[0, 1]]
    assert r.gate.tolist() == [[0.5, 0.5]]


def test_negative_zero_equals_positive_zero():
    s = np.array([[0.0, 0.0, 0.5]], np.float32)
    b = np.array([-0.0, 0.0, -0.5], np.float32)       # keys: -0, +0, 0.0
    r = routing.select(s, b, 2)
    assert r.idx.tolist() == [[0, 1]]


def test_sigmoid_against_mpmath():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    zs = [-745.0, -700.0, -40.0, -17.0, -3.5, -1e-9, 0.0, 1e-9, 0.3, 2.0, 16.6, 17.0, 40.0, 700.0]
    got = routing.sigmoid(np.array(zs))
    for z, g in zip(zs, got):
        ref = 1 / (1 + mpmath.exp(-mpmath.mpf(z)))
        assert abs(mpmath.mpf(g) - ref) <= 4e-16 * abs(ref) + mpmath.mpf(2) ** -1074


def test_logits_against_exact_rationals():
    rng = np.random.default_rng(11)
    u = rng.standard_normal((3, 24))
    e = rng.standard_normal((5, 24))
    z = routing.logits(u, e)
    for t in range(3):
        for i in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(c)) for a, c in zip(u[t], e[i]))
            bound = 24 * 2.0 ** -53 / (1 - 24 * 2.0 ** -53) * float(np.abs(u[t]) @ np.abs(e[i]))
            assert abs(float(Fraction(float(z[t, i])) - exact)) <= bound


def test_near_tie_gaps():
    s = np.array([[0.5, 0.5 + 2 ** -24, 0.25, 0.125]], np.float32)
    r = routing.select(s, np.zeros(4, np.float32), 1)
    kgap, ggap = routing.near_tie_gaps(r, 1, 1)
    assert 0 < kgap[0] < 1e-6 and ggap[0] == np.inf
    r = routing.select(s, np.zeros(4, np.float32), 2)
    kgap, _ = routing.near_tie_gaps(r, 2, 1)
    assert kgap[0] == (0.5 - 0.25) / 0.5
