"""Complementary sequence-wise balance loss: its forward value. Plain numpy, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the pwwt.cn study note on the DeepSeek-V3 Technical Report, §1.2
(complementary sequence-wise auxiliary loss) with §1.2.1-§1.2.3: the loss is
alpha times the sum over experts of f_i * P_i, where f_i is how often expert i
is actually selected within the sequence and P_i the probability that the
router prefers expert i within the sequence; alpha = 0.0001 (also in the
xyznot.com guides, "Método" §2). The page's formula image itself is missing,
so the normalisations are readings (listed in the design notes):
  B1 f_i = (number of the sequence's K_r * T_s selections that went to expert
     i) / (K_r * T_s), so sum_i f_i = 1; the selections are the router's
     actual (biased, group-limited) top-K;
  B2 P_i = mean over the sequence's tokens of s_{i,t} / sum_j s_{j,t}, the
     affinities normalised over all N_r routed experts (sum_i P_i = 1); a
     token whose affinities sum to 0 counts 1/N_r for every expert;
  B3 the batch is split into consecutive sequences of T_s tokens; each
     sequence has its own loss L = alpha * sum_i f_i P_i.
"""

import numpy as np

ALPHA = 1e-4


def seq_balance(s: np.ndarray, idx: np.ndarray, n_routed: int, top_k: int, seq_len: int,
                alpha: float = ALPHA):
    """Per-sequence (f [n_seq, N_r], P [n_seq, N_r], L [n_seq]) in fp64.

    s: [T, N_r] affinities (any float dtype, upcast exactly); idx: [T, K_r]
    selected experts; T must be a multiple of seq_len.
    """
    T = s.shape[0]
    if seq_len <= 0 or T % seq_len:
        raise ValueError("T must be a positive multiple of seq_len")
    n_seq = T // seq_len
    f = np.zeros((n_seq, n_routed))
    P = np.zeros((n_seq, n_routed))
    L = np.zeros(n_seq)
    for q in range(n_seq):
        rows = slice(q * seq_len, (q + 1) * seq_len)
        counts = np.bincount(np.asarray(idx[rows]).reshape(-1), minlength=n_routed)
        f[q] = counts / float(top_k * seq_len)
        sq = np.asarray(s[rows], dtype=np.float64)
        tot = sq.sum(axis=1, keepdims=True)
        norm = np.where(tot > 0, sq / np.where(tot > 0, tot, 1.0), 1.0 / n_routed)
        P[q] = norm.mean(axis=0)
        L[q] = alpha * float(np.dot(f[q], P[q]))
    return f, P, L
