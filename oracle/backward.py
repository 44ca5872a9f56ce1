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

from . import numerics as nx


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


# ----------------------------------------------------------------------------- FP8 layer
# The pages run all three GEMMs of a linear layer in E4M3 (pwwt.cn note section
# 3: Fprop, Dgrad and Wgrad in FP8, FP8 activations kept for the backward; the
# guides' key ideas: E4M3 everywhere, 1x128 activation tiles, 128x128 weight
# blocks). Readings where the pages stop (listed in the design notes):
#  * every GEMM input that is not a weight is quantised in tiles of 128 along
#    that GEMM's reduction dimension: Fprop and Dgrad inputs in 1x128 tiles
#    along their last axis; the two Wgrad inputs (the reduction runs over an
#    expert's rows) in 128x1 tiles along the rows, starting at the expert's
#    first row (a partial last tile holds the remaining rows);
#  * the weights are the layer's E4M3 weights (128x128 blocks), the same
#    values in Fprop and Dgrad; the weight gradient is taken with respect to
#    those values;
#  * the quantisers pass gradients straight through; everything else (router,
#    gates, SwiGLU) is differentiated exactly, in fp64.

def q_rows(x):
    """1x128 tiles along the last axis: E4M3 quantise-dequantise, fp64 -> fp64."""
    x = np.asarray(x, np.float64)
    return nx.dequant_act(*nx.quant_act_1x128(x.astype(np.float32)))


def q_cols(x):
    """128x1 tiles along the rows (from row 0; the last tile may be partial)."""
    x = np.asarray(x, np.float64)
    n = x.shape[0]
    pad = (-n) % 128
    xt = np.concatenate([x, np.zeros((pad, x.shape[1]))], axis=0).T
    return q_rows(xt).T[:n]


class _Fp8Linear(torch.autograd.Function):
    """y = st(Qr(st(x)) W^T) for W on the E4M3 grid; backward as the FP8 Dgrad
    dx = st(Qr(st(dy)) W) and Wgrad dW = Qc(st(dy))^T Qc(st(x)). st is the storage
    rounding of the tensors around the GEMMs (the identity, or bf16); the rounding
    passes gradients straight through, like the quantisers."""

    @staticmethod
    def forward(ctx, x, w, qr, qc, st):
        xs = torch.from_numpy(st(x.detach().numpy()))
        ctx.save_for_backward(xs, w)
        ctx.qr, ctx.qc, ctx.st = qr, qc, st
        return torch.from_numpy(st((torch.from_numpy(qr(xs.numpy())) @ w.T).detach().numpy()))

    @staticmethod
    def backward(ctx, dy):
        xs, w = ctx.saved_tensors
        dyn, xn = ctx.st(dy.detach().numpy()), xs.detach().numpy()
        dx = torch.from_numpy(ctx.st((torch.from_numpy(ctx.qr(dyn)) @ w).numpy()))
        dw = torch.from_numpy(ctx.qc(dyn)).T @ torch.from_numpy(ctx.qc(xn))
        return dx, dw, None, None, None


def _swiglu_fp8(x, w13, w2, qr, qc, st):
    inter = w13.shape[0] // 2
    ab = _Fp8Linear.apply(x, w13, qr, qc, st)
    a, v = ab[:, :inter], ab[:, inter:]
    return _Fp8Linear.apply(a * torch.sigmoid(a) * v, w2, qr, qc, st)


def _rules(quantise, store):
    ident = (lambda a: np.asarray(a, np.float64))
    qr, qc = (q_rows, q_cols) if quantise else (ident, ident)
    if store not in (None, "bf16"):
        raise ValueError("store must be None or 'bf16'")
    return qr, qc, (nx.bf16_round_f64 if store == "bf16" else ident)


def layer_grads_fp8(u64, e64, idx, dout64, w13q, w2q, w13sq=(), w2sq=(), experts=None, quantise=True,
                    store=None):
    """layer_grads for the FP8 layer: w13q / w2q (mappings expert -> fp64 arrays)
    and w13sq / w2sq are the E4M3 weights (ffn.fp8_weights of the masters); each
    expert's rows go through the FP8 GEMMs above. quantise=False replaces every
    quantiser by the identity, which must give layer_grads on the same weights.
    store="bf16" rounds to bf16 every tensor a GEMM reads before quantising it and
    every Fprop and Dgrad output (the pages' GEMMs take FP8 inputs and give BF16 or
    FP32 results: pwwt.cn note section 3); None keeps them in fp64."""
    qr, qc, st = _rules(quantise, store)
    u = torch.tensor(u64, dtype=torch.float64, requires_grad=True)
    E = torch.tensor(e64, dtype=torch.float64, requires_grad=True)
    idx_t = torch.tensor(np.asarray(idx), dtype=torch.long)
    used = sorted(set(np.asarray(idx).reshape(-1).tolist()))
    want = used if experts is None else sorted(experts)
    W13 = {e: torch.tensor(w13q[e], dtype=torch.float64, requires_grad=e in want) for e in used}
    W2 = {e: torch.tensor(w2q[e], dtype=torch.float64, requires_grad=e in want) for e in used}
    W13s = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in w13sq]
    W2s = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in w2sq]

    s = torch.sigmoid(u @ E.T)
    sel = torch.gather(s, 1, idx_t)
    g = sel / sel.sum(dim=1, keepdim=True)
    out = u
    for a, b in zip(W13s, W2s):
        out = out + _swiglu_fp8(u, a, b, qr, qc, st)
    routed = torch.zeros_like(u)
    for e in used:
        rows, ks = np.nonzero(np.asarray(idx) == e)     # rows in token order
        rows_t, ks_t = torch.tensor(rows), torch.tensor(ks)
        y = _swiglu_fp8(u[rows_t], W13[e], W2[e], qr, qc, st)
        routed = routed.index_add(0, rows_t, g[rows_t, ks_t][:, None] * y)
    out = out + routed
    (out * torch.tensor(dout64, dtype=torch.float64)).sum().backward()
    return {
        "du": u.grad.numpy(), "dE": E.grad.numpy(),
        "dw13": {e: W13[e].grad.numpy() for e in want}, "dw2": {e: W2[e].grad.numpy() for e in want},
        "dw13s": [w.grad.numpy() for w in W13s], "dw2s": [w.grad.numpy() for w in W2s],
    }


def expert_weight_grads_fp8(u_rows64, gate_rows64, dout_rows64, w13q, w2q, quantise=True, store=None):
    """expert_weight_grads for one routed expert of the FP8 layer: the rows that chose it
    (u [n, d], in token order, the order its 128-row Wgrad tiles follow), their gates and
    upstream gradients, and its E4M3 weights (fp64 values). Equal to layer_grads_fp8's
    dw13[e], dw2[e] (pinned against it) without the other experts; quantise and store as
    there."""
    qr, qc, st = _rules(quantise, store)
    u = torch.tensor(u_rows64, dtype=torch.float64)
    W13 = torch.tensor(w13q, dtype=torch.float64, requires_grad=True)
    W2 = torch.tensor(w2q, dtype=torch.float64, requires_grad=True)
    g = torch.tensor(np.asarray(gate_rows64, dtype=np.float64))[:, None]
    out = g * _swiglu_fp8(u, W13, W2, qr, qc, st)
    (out * torch.tensor(dout_rows64, dtype=torch.float64)).sum().backward()
    return W13.grad.numpy(), W2.grad.numpy()
