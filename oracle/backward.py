"""Backward pass of the DeepSeekMoE layer for a fixed routing, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward is the output equation of the xyznot.com guides ("Método" §2),
h'_t = u_t + sum_s FFN^(s)_s(u_t) + sum_k g_{k,t} FFN^(r)_{idx_k}(u_t), with
s = Sigmoid(u E^T), g = s_sel / sum(s_sel) over the selected experts, and the
SwiGLU expert (reading R8). The selection (which experts) is piecewise
constant in u, E and b, so for a fixed selection the gradient flows through
the gates' dependence on s, and the bias receives none (pwwt.cn note
§1.1.2-§1.1.3: b only routes and is updated by the load rule). Given an
upstream gradient dout [T, d] this returns d(sum(out * dout)) with respect to
u, E and every expert's W13 / W2 (routed and shared).

Plain PyTorch CPU autograd in float64 is the library primitive here; the
tests pin it with central finite differences of the forward oracle.
"""

import numpy as np
import torch


def _swiglu(x, w13, w2):
    inter = w13.shape[0] // 2
    a = x @ w13[:inter].T
    v = x @ w13[inter:].T
    return (a * torch.sigmoid(a) * v) @ w2.T


def layer_grads(u64, e64, idx, dout64, w13, w2, w13s=(), w2s=(), experts=None):
    """Gradients of sum(out * dout) for the selection `idx` [T, K] (held fixed).

    u64 [T, d], e64 [N_r, d], dout64 [T, d]: fp64 arrays. w13 / w2: mappings
    expert -> fp64 [2I, d] / [d, I] covering every expert in idx. w13s / w2s:
    the shared experts' fp64 weights. `experts` limits which routed experts'
    weight gradients are returned (default: every expert in idx).
    Returns dict(du, dE, dw13 {e: ...}, dw2 {e: ...}, dw13s [...], dw2s [...]).
    """
    u = torch.tensor(u64, dtype=torch.float64, requires_grad=True)
    E = torch.tensor(e64, dtype=torch.float64, requires_grad=True)
    idx_t = torch.tensor(np.asarray(idx), dtype=torch.long)
    used = sorted(set(np.asarray(idx).reshape(-1).tolist()))
    want = used if experts is None else sorted(experts)
    W13 = {e: torch.tensor(w13[e], dtype=torch.float64, requires_grad=e in want) for e in used}
    W2 = {e: torch.tensor(w2[e], dtype=torch.float64, requires_grad=e in want) for e in used}
    W13s = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in w13s]
    W2s = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in w2s]

    s = torch.sigmoid(u @ E.T)
    sel = torch.gather(s, 1, idx_t)
    g = sel / sel.sum(dim=1, keepdim=True)
    out = u
    for a, b in zip(W13s, W2s):
        out = out + _swiglu(u, a, b)
    routed = torch.zeros_like(u)
    for e in used:
        rows, ks = np.nonzero(np.asarray(idx) == e)
        rows_t, ks_t = torch.tensor(rows), torch.tensor(ks)
        y = _swiglu(u[rows_t], W13[e], W2[e])
        routed = routed.index_add(0, rows_t, g[rows_t, ks_t][:, None] * y)
    out = out + routed
    (out * torch.tensor(dout64, dtype=torch.float64)).sum().backward()
    return {
        "du": u.grad.numpy(), "dE": E.grad.numpy(),
        "dw13": {e: W13[e].grad.numpy() for e in want}, "dw2": {e: W2[e].grad.numpy() for e in want},
        "dw13s": [w.grad.numpy() for w in W13s], "dw2s": [w.grad.numpy() for w in W2s],
    }


def expert_weight_grads(u_rows64, gate_rows64, dout_rows64, w13_64, w2_64):
    """One routed expert's weight gradients: the rows that chose it (u [n, d]), their gates
    g [n] and upstream gradients dout [n, d]. The expert enters out only through g * FFN(u),
    so these equal layer_grads' dw13[e], dw2[e] (pinned against it) without the other
    experts. Returns (dw13 [2I, d], dw2 [d, I]) fp64."""
    u = torch.tensor(u_rows64, dtype=torch.float64)
    W13 = torch.tensor(w13_64, dtype=torch.float64, requires_grad=True)
    W2 = torch.tensor(w2_64, dtype=torch.float64, requires_grad=True)
    g = torch.tensor(np.asarray(gate_rows64, dtype=np.float64))[:, None]
    out = g * _swiglu(u, W13, W2)
    (out * torch.tensor(dout_rows64, dtype=torch.float64)).sum().backward()
    return W13.grad.numpy(), W2.grad.numpy()
