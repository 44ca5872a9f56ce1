"""Dispatch layout of the routed rows (single-GPU analog of the pages' dispatch).

The pwwt.cn note §4 describes dispatch (tokens sent to the devices holding
their experts) and combine (outputs returned and summed with the gates). On one
GPU the analog is a permutation that groups the T*K (token, expert) rows by
expert, with no capacity limit (note §1.4: no token dropping).

Layout reading (the pages give none): rows of expert e occupy
[offsets[e], offsets[e+1]), offsets = exclusive scan of the per-expert loads;
inside an expert, rows are in ascending token order; row_token[r] is the token
of permuted row r; slot_row[t*K + k] is the permuted row of (t, idx[t, k]).
"""

import numpy as np


def layout(idx: np.ndarray, n_routed: int):
    T, K = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=n_routed).astype(np.int64)
    offsets = np.zeros(n_routed + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_token = np.empty(T * K, dtype=np.int64)
    slot_row = np.empty(T * K, dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(T):                      # ascending token order within each expert
        for k in range(K):
            e = idx[t, k]
            r = fill[e]
            fill[e] += 1
            row_token[r] = t
            slot_row[t * K + k] = r
    return offsets, row_token, slot_row


def layout_fast(idx: np.ndarray, n_routed: int):
    """Same result as `layout`, vectorised (a stable sort by expert)."""
    T, K = idx.shape
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")      # flat index t*K+k ascends -> token ascends
    counts = np.bincount(flat, minlength=n_routed).astype(np.int64)
    offsets = np.zeros(n_routed + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_token = (order // K).astype(np.int64)
    slot_row = np.empty(T * K, dtype=np.int64)
    slot_row[order] = np.arange(T * K)
    return offsets, row_token, slot_row
