"""Pins of oracle.balance (the sequence-wise balance loss value) against values
fixed outside it: hand-computed fractions (tests/golden/balance_cases.json),
closed forms and invariants that follow from the definition."""

import json
import os

import numpy as np
import pytest

from oracle import balance

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "balance_cases.json")


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"][:3])
def test_hand_cases(case):
    s = np.array(case["s"], dtype=np.float32)
    idx = np.array(case["idx"], dtype=np.int32)
    f, P, L = balance.seq_balance(s, idx, case["n_routed"], case["top_k"], case["seq_len"], case["alpha"])
    assert np.array_equal(f, np.array(case["f"]))
    assert np.array_equal(P, np.array(case["P"]))
    assert np.allclose(L, case["alpha"] * np.array(case["sum_fP"]), rtol=1e-15, atol=0)


def _rand(seed, T, N, K):
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.0, 1.0, (T, N)).astype(np.float32)
    idx = np.stack([rng.choice(N, K, replace=False) for _ in range(T)]).astype(np.int32)
    return s, idx


def test_balanced_selection_closed_form():
    """Every expert selected equally often: f_i = 1/N, so L = alpha/N whatever the affinities."""
    N, K, Ts = 16, 4, 64
    rng = np.random.default_rng(1)
    s = rng.uniform(0, 1, (Ts, N)).astype(np.float32)
    idx = np.array([[(4 * t + k) % N for k in range(K)] for t in range(Ts)], dtype=np.int32)
    f, P, L = balance.seq_balance(s, idx, N, K, Ts)
    assert np.allclose(f, 1.0 / N, rtol=0, atol=1e-15)
    assert np.isclose(L[0], balance.ALPHA / N, rtol=1e-12)


def test_uniform_affinity_closed_form():
    """Equal affinities in every row: P_i = 1/N, so L = alpha/N whatever the selection."""
    N, K, Ts = 32, 8, 40
    _, idx = _rand(2, Ts, N, K)
    s = np.full((Ts, N), 0.3, dtype=np.float32)
    f, P, L = balance.seq_balance(s, idx, N, K, Ts)
    assert np.allclose(P, 1.0 / N, rtol=1e-12)
    assert np.isclose(L[0], balance.ALPHA / N, rtol=1e-12)


def test_collapse_case():
    """All tokens pick experts 0..K-1 and put all their affinity there (equally): f_i = P_i = 1/K
    on those experts, so L = alpha/K -- the largest value the loss can take."""
    N, K, Ts = 16, 4, 10
    s = np.zeros((Ts, N), dtype=np.float32)
    s[:, :K] = 0.5
    idx = np.tile(np.arange(K, dtype=np.int32), (Ts, 1))
    _, _, L = balance.seq_balance(s, idx, N, K, Ts)
    assert np.isclose(L[0], balance.ALPHA / K, rtol=1e-12)


def test_invariants():
    N, K, Ts, n_seq = 24, 6, 50, 3
    s, idx = _rand(3, Ts * n_seq, N, K)
    f, P, L = balance.seq_balance(s, idx, N, K, Ts)
    assert np.allclose(f.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # L <= alpha * max f and L <= alpha * max P (a weighted mean of the other vector)
    assert (L <= balance.ALPHA * f.max(axis=1) + 1e-18).all()
    assert (L <= balance.ALPHA * P.max(axis=1) + 1e-18).all()
    # relabelling the experts consistently changes nothing
    perm = np.random.default_rng(4).permutation(N)
    inv = np.argsort(perm)
    f2, P2, L2 = balance.seq_balance(s[:, perm], inv[idx].astype(np.int32), N, K, Ts)
    assert np.allclose(L2, L, rtol=1e-13)
    assert np.allclose(f2, f[:, perm]) and np.allclose(P2, P[:, perm])
    # scaling a token's affinities leaves P unchanged; the order of a token's selections too
    s3 = s.copy()
    s3[5] *= 4.0
    _, P3, _ = balance.seq_balance(s3, idx[:, ::-1].copy(), N, K, Ts)
    assert np.allclose(P3, P, rtol=1e-13)
    # sequences are independent: each sequence alone gives its own value
    for q in range(n_seq):
        rows = slice(q * Ts, (q + 1) * Ts)
        _, _, Lq = balance.seq_balance(s[rows], idx[rows], N, K, Ts)
        assert Lq[0] == L[q]


def test_zero_row_counts_uniform():
    N, K, Ts = 8, 2, 2
    s = np.zeros((Ts, N), dtype=np.float32)
    s[1, 3] = 1.0
    idx = np.array([[0, 1], [3, 4]], dtype=np.int32)
    _, P, _ = balance.seq_balance(s, idx, N, K, Ts)
    want = np.full(N, 0.5 / N)
    want[3] += 0.5
    assert np.allclose(P[0], want, rtol=0, atol=1e-15)


def test_bad_seq_len():
    s, idx = _rand(5, 10, 8, 2)
    with pytest.raises(ValueError):
        balance.seq_balance(s, idx, 8, 2, 3)
