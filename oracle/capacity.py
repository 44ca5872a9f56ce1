"""Capacity-limited routing with token dropping: the DeepSeek-V2-style baseline
that the DeepSeek-V3 method does without. Plain numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the pwwt.cn study note on the DeepSeek-V3 Technical Report, §1.4 (no
token dropping): V2 sets a compute budget, and when a device receives more
tokens than it, sorts them by affinity and drops the lowest-scoring ones,
which then skip that layer's FFN; V3 drops none. Readings (design notes):
  C1 on one GPU the budget is per expert: capacity C = ceil(cf * T * K / N_r)
     (T*K/N_r is the mean load, cf the capacity factor);
  C2 an expert with more than C selections keeps the C with the largest
     affinity s_{i,t} (the unbiased score), ties to the lower token index;
  C3 a dropped selection contributes nothing: the token's other gates are not
     renormalised (out = u + shared + sum over kept k of g_k y_k).
"""

import math

import numpy as np


def capacity(T: int, K: int, n_routed: int, cf: float) -> int:
    return int(math.ceil(cf * T * K / n_routed))


def keep_mask(s, idx, n_routed: int, cap: int) -> np.ndarray:
    """keep [T, K] bool: for each expert, its `cap` selections with the largest
    affinity s[t, e] (ties: lower token first); every selection when it has <= cap."""
    idx = np.asarray(idx)
    T, K = idx.shape
    keep = np.ones((T, K), dtype=bool)
    for e in range(n_routed):
        ts, ks = np.nonzero(idx == e)
        if len(ts) <= cap:
            continue
        order = sorted(range(len(ts)), key=lambda i: (-float(s[ts[i], e]), int(ts[i])))
        for i in order[cap:]:
            keep[ts[i], ks[i]] = False
    return keep


def dropped_gates(gate, keep) -> np.ndarray:
    """Reading C3: the gate of a dropped selection becomes 0 and the kept gates stay as routed,
    so the layer output (oracle.ffn.layer with these gates) is u + shared + the kept terms."""
    return np.where(np.asarray(keep, dtype=bool), np.asarray(gate, dtype=np.float64), 0.0)
