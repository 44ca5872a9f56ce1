"""Expert FFNs and the layer output, fp64.

Output equation (xyznot.com guides, "Método" §2):
    h'_t = u_t + sum_{i<=N_s} FFN^(s)_i(u_t) + sum_{i<=N_r} g_{i,t} FFN^(r)_i(u_t)
The pages never state the FFN's inner form. Reading taken: SwiGLU without
biases, FFN(x) = W2 (SiLU(W1 x) * (W3 x)), SiLU(a) = a * sigmoid(a); W13 stacks
W1 (rows 0..I-1) over W3 (rows I..2I-1). Each shared expert has its own weights.
No token is dropped (pwwt.cn note §1.4): every (token, selected expert) pair is
evaluated, with no capacity limit.

FP8 diagnostic ("oracle B"): the same layer on E4M3-dequantised u, H and W with
the pages' 1x128 / 128x128 scaling (xyznot.com guides, FP8 key idea; pwwt.cn
note §3), to separate quantisation error from kernel error. u is quantised
once, in 1x128 tiles along d; H in 1x128 tiles along I inside each expert;
W13 and W2 in 128x128 blocks. Pinned against an independent construction with
torch's float8_e4m3fn cast (tests/test_oracle_ffn.py).
"""

import numpy as np

from . import numerics as nx
from . import routing as rt


def _sig(a):
    return rt.sigmoid(a)


def swiglu(x64: np.ndarray, w13_64: np.ndarray, w2_64: np.ndarray) -> np.ndarray:
    """One expert: [R, d] -> [R, d], all fp64."""
    inter = w13_64.shape[0] // 2
    a = x64 @ w13_64[:inter].T
    v = x64 @ w13_64[inter:].T
    h = a * _sig(a) * v
    return h @ w2_64.T


def _w64(arr, dtype):
    return nx.to_f64(arr, dtype)


def layer(cfg, u, idx, gate64, w13, w2, w13s, w2s, tokens=None, wdtype=None,
          fp8=False, weights=None):
    """Layer output for `tokens` (default all): u + shared + sum_k g_k y_k (fp64).

    u, weights: canonical input arrays (bf16 bits or fp32). idx/gate64: routing.
    Experts are converted to fp64 one at a time. Returns [len(tokens), d] fp64.
    With fp8=True, u, H and the weights go through E4M3 quantise-dequantise.

    weights: optional callable (kind, i) -> (w13, w2) for kind "shared" or
    "routed", returning the expert's fp64 weights as the layer uses them (for
    fp8, already through fp8_weights); then w13/w2/w13s/w2s are not read. It
    lets a caller prepare experts ahead (for example on other threads) without
    changing what is computed. Experts are used in ascending order.
    """
    wdtype = wdtype or ("bf16" if cfg.expert_dtype == "bf16" else "f32")

    def expert_w(kind, i):
        if weights is not None:
            return weights(kind, i)
        a, b = (w13s[i], w2s[i]) if kind == "shared" else (w13[i], w2[i])
        a, b = _w64(a, wdtype), _w64(b, wdtype)
        return fp8_weights(a, b) if fp8 else (a, b)

    T = u.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    u64 = nx.to_f64(u[tok], cfg.in_dtype)
    if fp8:
        xq = _fp8_act(u64)
    else:
        xq = u64
    out = u64.copy()
    for s in range(cfg.n_shared):
        out += _expert(xq, *expert_w("shared", s), fp8)
    sub_idx = idx[tok]
    sub_gate = gate64[tok]
    for e in np.unique(sub_idx):
        rows, ks = np.nonzero(sub_idx == e)
        y = _expert(xq[rows], *expert_w("routed", int(e)), fp8)
        out[rows] += sub_gate[rows, ks][:, None] * y
    return out


def fp8_weights(w13_64, w2_64):
    """One expert's weights through E4M3 with one fp32 scale per 128x128 block
    (W13 [2I, d] and W2 [d, I] each blocked on its own), back to fp64."""
    c13, s13 = nx.quant_w_128x128(w13_64.astype(np.float32))
    c2, s2 = nx.quant_w_128x128(w2_64.astype(np.float32))
    return nx.dequant_w(c13, s13), nx.dequant_w(c2, s2)


def _fp8_act(x64):
    codes, scale = nx.quant_act_1x128(x64.astype(np.float32))
    return nx.dequant_act(codes, scale)


def _expert(x64, w13_64, w2_64, fp8):
    """One expert on rows x64. fp8: the weights are already E4M3-dequantised
    (fp8_weights); H is quantised here, in 1x128 tiles along I."""
    if not fp8:
        return swiglu(x64, w13_64, w2_64)
    inter = w13_64.shape[0] // 2
    a = x64 @ w13_64[:inter].T
    v = x64 @ w13_64[inter:].T
    h = a * _sig(a) * v
    return _fp8_act(h) @ w2_64.T
