"""Brute-force group-limited top-K by enumeration with exact rationals.

An independent check of `routing.select` for small inputs: instead of sorting,
enumerate every set of M groups and every K-subset of their experts and keep
the set with the largest exact sum (fractions.Fraction of the fp32 values, so
summation order cannot matter). Among equal sums the lexicographically smallest
sorted index tuple wins, which is the (value desc, index asc) rule of the
sorted selection. Only the group score keeps its fp32 rounding: it is the fp32
sequential sum (largest first) of the group's q largest keys, as the selection
defines it (pwwt.cn note §1.3: nodes ranked by the sum of their top K_r/M
scores; the sum's precision is a reading, see routing.py R2).
"""

from fractions import Fraction
from itertools import combinations

import numpy as np


def _best_subset(values, items, k):
    best, best_sum = None, None
    for sub in combinations(sorted(items), k):
        ssum = sum(Fraction(float(values[i])) for i in sub)
        if best is None or ssum > best_sum or (ssum == best_sum and sub < best):
            best, best_sum = sub, ssum
    return best


def _group_score(gkeys32, q):
    top = _best_subset(gkeys32, range(len(gkeys32)), q)
    vals = sorted((np.float32(gkeys32[i]) for i in top), reverse=True)
    acc = np.float32(vals[0])
    for v in vals[1:]:
        acc = np.float32(acc + v)
    return acc


def select_one(s32_row, b32, top_k, n_groups=1, topk_groups=1, group_topk=None,
               group_score_biased=1):
    """One token: (sorted expert index tuple, chosen group tuple)."""
    s32_row = np.asarray(s32_row, dtype=np.float32)
    N = s32_row.shape[0]
    k32 = np.asarray([np.float32(s32_row[i] + np.float32(b32[i])) for i in range(N)], dtype=np.float32)
    if n_groups > 1:
        q = group_topk if group_topk is not None else top_k // topk_groups
        size = N // n_groups
        src = k32 if group_score_biased else s32_row
        gs = [_group_score(src[g * size:(g + 1) * size], q) for g in range(n_groups)]
        groups = _best_subset(gs, range(n_groups), topk_groups)
        cand = [g * size + j for g in groups for j in range(size)]
    else:
        groups = (0,)
        cand = list(range(N))
    experts = _best_subset(k32, cand, top_k)
    return experts, groups
