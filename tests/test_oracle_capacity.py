"""Pins of oracle.capacity (the token-dropping baseline's selection)."""

import numpy as np

from oracle import capacity


def test_capacity_value():
    assert capacity.capacity(8192, 8, 256, 1.0) == 256
    assert capacity.capacity(8192, 8, 256, 1.25) == 320
    assert capacity.capacity(10, 3, 7, 1.0) == 5          # ceil(30/7)


def test_hand_case():
    # expert 0 is chosen by tokens 0..4 (capacity 3): s = .9, .5, .7, .5, .1 -> keep 0, 2, and
    # of the tied .5 the lower token (1); tokens 3 and 4 drop their expert-0 selection.
    s = np.array([[.9, .1], [.5, .2], [.7, .3], [.5, .4], [.1, .8]], dtype=np.float32)
    idx = np.array([[0, 1], [0, 1], [0, 1], [0, 1], [0, 1]])
    keep = capacity.keep_mask(s, idx, 2, 3)
    assert keep[:, 0].tolist() == [True, True, True, False, False]
    # expert 1 (second column): s = .1 .2 .3 .4 .8 -> keep tokens 4, 3, 2
    assert keep[:, 1].tolist() == [False, False, True, True, True]


def test_invariants():
    rng = np.random.default_rng(0)
    T, K, N = 300, 4, 16
    s = rng.uniform(0, 1, (T, N)).astype(np.float32)
    idx = np.stack([rng.choice(N, K, replace=False, p=np.linspace(1, 3, N) / np.linspace(1, 3, N).sum())
                    for _ in range(T)])
    for cf in (0.5, 1.0, 1.25, 10.0):
        cap = capacity.capacity(T, K, N, cf)
        keep = capacity.keep_mask(s, idx, N, cap)
        for e in range(N):
            sel = idx == e
            kept = keep & sel
            assert kept.sum() == min(cap, sel.sum())
            # every kept selection's affinity >= every dropped one's of the same expert
            if (sel & ~keep).any():
                assert s[np.nonzero(kept)[0], e].min() >= s[np.nonzero(sel & ~keep)[0], e].max()
        if cf >= 10.0:
            assert keep.all()


def test_dropped_gates_zero_only_dropped():
    g = np.array([[.5, .3, .2], [.6, .4, 0.]])
    keep = np.array([[True, False, True], [False, False, True]])
    out = capacity.dropped_gates(g, keep)
    assert out.tolist() == [[.5, 0., .2], [0., 0., 0.]]
    # a kept gate is the routed one, unchanged (no renormalisation over the kept set)
    assert out[0, 0] == g[0, 0] and out[0].sum() < 1.0
