"""Pins of the dispatch layout: it is a permutation of the T*K rows, grouped by
expert at the offsets of the exclusive scan of the loads, ascending token order
inside each expert, and slot_row / row_token are mutually inverse."""

import numpy as np
import pytest

from oracle import permute


@pytest.mark.parametrize("T,N,K", [(1, 4, 1), (17, 8, 3), (64, 16, 4), (300, 64, 6)])
def test_layout_properties(T, N, K):
    rng = np.random.default_rng(T * N + K)
    idx = np.stack([rng.choice(N, K, replace=False) for _ in range(T)])
    offsets, row_token, slot_row = permute.layout(idx, N)
    counts = np.bincount(idx.reshape(-1), minlength=N)
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all() and offsets[-1] == T * K
    assert sorted(slot_row.tolist()) == list(range(T * K))
    for t in range(T):
        for k in range(K):
            r = slot_row[t * K + k]
            assert row_token[r] == t
            e = idx[t, k]
            assert offsets[e] <= r < offsets[e + 1]
    for e in range(N):
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()
    o2, r2, s2 = permute.layout_fast(idx, N)
    assert (o2 == offsets).all() and (r2 == row_token).all() and (s2 == slot_row).all()


def test_layout_skewed_loads():
    T, N, K = 50, 8, 2
    idx = np.tile(np.array([[0, 1]]), (T, 1))
    offsets, row_token, slot_row = permute.layout(idx, N)
    assert offsets.tolist() == [0, 50, 100, 100, 100, 100, 100, 100, 100]
    assert row_token.tolist() == list(range(50)) * 2
