"""Router of the DeepSeekMoE layer: affinities, biased group-limited top-K,
normalised gates, per-expert loads and the bias update. Plain numpy.

Sources (DeepSeek-V3 Technical Report pages):
  * xyznot.com guides (ar/pt), "Método" §2: s_{i,t} = Sigmoid(u_t^T e_i);
    g'_{i,t} = s_{i,t} if s_{i,t}+b_i is in Topk({s_{j,t}+b_j}, K_r), else 0;
    g_{i,t} = g'_{i,t} normalised; b_i -/+ gamma, gamma = 0.001.
  * pwwt.cn note §1.1.2: the bias only decides *who* is selected; gates use the
    original s (step 3). §1.1.3: per-step load of the whole batch, then
    b_i <- b_i - gamma if overloaded, + gamma if underloaded.
  * pwwt.cn note §1.3 (and the szhzxw.cn page, "节点限制路由"): a token goes to at
    most M nodes, ranked by the sum of the top K_r/M affinity scores of the
    experts on each node.

Readings where the pages are silent (each listed in the design notes):
  R1 group g = experts [g*N_r/G, (g+1)*N_r/G) (contiguous blocks);
  R2 group score = fp32 sequential sum, in descending order, of the group's top
     q = K_r/M keys; with group_score_biased=1 the keys are s+b (routing
     decisions look at the biased score), with 0 they are s;
  R3 exactly K_r experts; total order (key desc, expert index asc); groups by
     (score desc, group index asc); -0 == +0;
  R4 idx is returned in that rank order;
  R5 gates over the K_r selected, no extra scale; a zero sum gives 1/K_r;
  R6 overloaded: c_i > T*K_r/N_r, underloaded: c_i < T*K_r/N_r, otherwise no
     change (integer comparison N_r*c_i vs T*K_r); b stays fp32, one fp32 add
     of fl32(gamma) per step.
"""

from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------- affinities
def logits(u64: np.ndarray, e64: np.ndarray, block: int = 2048) -> np.ndarray:
    """z = u E^T in fp64, computed in row blocks (a library matmul per block)."""
    z = np.empty((u64.shape[0], e64.shape[0]), dtype=np.float64)
    for r in range(0, u64.shape[0], block):
        z[r:r + block] = u64[r:r + block] @ e64.T
    return z


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1/(1+exp(-z)), evaluated as exp(z)/(1+exp(z)) for z < 0 (no overflow)."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def keys(s32: np.ndarray, b32: np.ndarray) -> np.ndarray:
    """Routing key fl32(s + b): one IEEE binary32 addition."""
    return (np.asarray(s32, dtype=np.float32) + np.asarray(b32, dtype=np.float32)[None, :]).astype(np.float32)


# ----------------------------------------------------------------- selection
def group_scores(k32: np.ndarray, n_groups: int, q: int) -> np.ndarray:
    """[T, G] fp32: sequential fp32 sum of each group's q largest values, largest first."""
    T, N = k32.shape
    g = np.asarray(k32, dtype=np.float32).reshape(T, n_groups, N // n_groups)
    top = -np.sort(-g, axis=2)[:, :, :q]
    acc = top[:, :, 0].astype(np.float32)
    for j in range(1, q):
        acc = (acc + top[:, :, j]).astype(np.float32)
    return acc


def _order_desc(vals: np.ndarray) -> np.ndarray:
    """Per row: indices sorted by (value desc, index asc). -0 and +0 compare equal."""
    return np.argsort(-np.asarray(vals, dtype=np.float64), axis=1, kind="stable")


@dataclass
class Route:
    idx: np.ndarray          # [T, K] int64, rank order
    gate: np.ndarray         # [T, K] fp64
    counts: np.ndarray       # [N_r] int64
    key: np.ndarray          # [T, N_r] fp32
    cand: np.ndarray         # [T, N_r] bool, experts inside the chosen groups
    gscore: np.ndarray       # [T, G] fp32 (zeros when G == 1)
    groups: np.ndarray       # [T, M] int64 chosen groups, rank order


def select(s32, b32, top_k, n_groups=1, topk_groups=1, group_topk=None,
           group_score_biased=1, s_gate=None) -> Route:
    """Group-limited top-K on fl32(s + b); gates from the unbiased s.

    s32: [T, N_r] fp32 affinities (the values the selection compares).
    s_gate: values the gates are normalised from (defaults to s32; the
            end-to-end oracle passes its fp64 affinities).
    """
    s32 = np.asarray(s32, dtype=np.float32)
    T, N = s32.shape
    k32 = keys(s32, b32)
    if n_groups > 1:
        q = group_topk if group_topk is not None else top_k // topk_groups
        gsrc = k32 if group_score_biased else s32
        gs = group_scores(gsrc, n_groups, q)
        groups = _order_desc(gs)[:, :topk_groups]
        size = N // n_groups
        gmask = np.zeros((T, n_groups), dtype=bool)
        np.put_along_axis(gmask, groups, True, axis=1)
        cand = np.repeat(gmask, size, axis=1)
    else:
        gs = np.zeros((T, 1), dtype=np.float32)
        groups = np.zeros((T, 1), dtype=np.int64)
        cand = np.ones((T, N), dtype=bool)
    masked = np.where(cand, k32.astype(np.float64), -np.inf)
    idx = _order_desc(masked)[:, :top_k]
    sg = s32.astype(np.float64) if s_gate is None else np.asarray(s_gate, dtype=np.float64)
    sel = np.take_along_axis(sg, idx, axis=1)
    tot = sel.sum(axis=1, keepdims=True)
    gate = np.where(tot > 0, sel / np.where(tot > 0, tot, 1.0), 1.0 / top_k)
    counts = np.bincount(idx.reshape(-1), minlength=N).astype(np.int64)
    assert counts.sum() == T * top_k
    return Route(idx=idx.astype(np.int64), gate=gate, counts=counts, key=k32,
                 cand=cand, gscore=gs, groups=groups.astype(np.int64))


# ----------------------------------------------------------------- balancing
def bias_step(counts: np.ndarray, b32: np.ndarray, T: int, top_k: int, gamma: float = 0.001) -> np.ndarray:
    """End-of-step update: b_i - gamma if c_i > mean load, + gamma if below, else unchanged."""
    c = np.asarray(counts, dtype=np.int64)
    n = c.shape[0]
    delta = np.sign(T * top_k - n * c)                 # exact integer comparison with the mean
    b = np.asarray(b32, dtype=np.float32)
    g32 = np.float32(gamma)
    stepped = (b + delta.astype(np.float32) * g32).astype(np.float32)
    return np.where(delta != 0, stepped, b).astype(np.float32)


# ----------------------------------------------------------------- near ties
def near_tie_gaps(route: Route, top_k: int, topk_groups: int):
    """Relative gaps (K-th vs (K+1)-th candidate key; M-th vs (M+1)-th group score).

    rel = (v_K - v_{K+1}) / max(|v_K|, |v_{K+1}|); +inf when there is no
    (K+1)-th value. A token whose gap is below the end-to-end threshold may
    legitimately route differently under a different (correct) rounding of u.E.
    """
    T = route.key.shape[0]
    masked = np.where(route.cand, route.key.astype(np.float64), -np.inf)
    srt = -np.sort(-masked, axis=1)
    kgap = np.full(T, np.inf)
    if srt.shape[1] > top_k:
        a, b = srt[:, top_k - 1], srt[:, top_k]
        ok = np.isfinite(b)
        den = np.maximum(np.abs(a), np.abs(b))
        kgap[ok] = np.where(den[ok] > 0, (a[ok] - b[ok]) / np.where(den[ok] > 0, den[ok], 1), 0.0)
    ggap = np.full(T, np.inf)
    G = route.gscore.shape[1]
    if G > topk_groups:
        gs = -np.sort(-route.gscore.astype(np.float64), axis=1)
        a, b = gs[:, topk_groups - 1], gs[:, topk_groups]
        den = np.maximum(np.abs(a), np.abs(b))
        ggap = np.where(den > 0, (a - b) / np.where(den > 0, den, 1), 0.0)
    return kgap, ggap


def route_tokens(u64, e64, b32, cfg, s_mode="e2e") -> tuple:
    """End-to-end routing from fp64 logits: returns (Route, s64, s32)."""
    z = logits(u64, e64)
    s64 = sigmoid(z)
    s32 = s64.astype(np.float32)
    r = select(s32, b32, cfg.top_k, cfg.n_groups, cfg.topk_groups, cfg.group_topk,
               cfg.group_score_biased, s_gate=s64 if s_mode == "e2e" else None)
    return r, s64, s32
