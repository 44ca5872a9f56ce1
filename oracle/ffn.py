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
          fp8=False):
    """Layer output for `tokens` (default all): u + shared + sum_k g_k y_k (fp64).

    u, weights: canonical input arrays (bf16 bits or fp32). idx/gate64: routing.
    Experts are converted to fp64 one at a time. Returns [len(tokens), d] fp64.
    With fp8=True, u, H and the weights go through E4M3 quantise-dequantise.
    """
    wdtype = wdtype or ("bf16" if cfg.expert_dtype == "bf16" else "f32")
    T = u.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    u64 = nx.to_f64(u[tok], cfg.in_dtype)
    if fp8:
        xq = _fp8_act(u64)
    else:
        xq = u64
    out = u64.copy()
    for s in range(cfg.n_shared):
        out += _expert(xq, _w64(w13s[s], wdtype), _w64(w2s[s], wdtype), fp8)
    sub_idx = idx[tok]
    sub_gate = gate64[tok]
    for e in np.unique(sub_idx):
        rows, ks = np.nonzero(sub_idx == e)
        y = _expert(xq[rows], _w64(w13[e], wdtype), _w64(w2[e], wdtype), fp8)
        out[rows] += sub_gate[rows, ks][:, None] * y
    return out


def _fp8_act(x64):
    codes, scale = nx.quant_act_1x128(x64.astype(np.float32))
    return nx.dequant_act(codes, scale)


def _expert(x64, w13_64, w2_64, fp8):
    if not fp8:
        return swiglu(x64, w13_64, w2_64)
    inter = w13_64.shape[0] // 2
    c13, s13 = nx.quant_w_128x128(w13_64.astype(np.float32))
    c2, s2 = nx.quant_w_128x128(w2_64.astype(np.float32))
    w13q = nx.dequant_w(c13, s13)
    w2q = nx.dequant_w(c2, s2)
    a = x64 @ w13q[:inter].T
    v = x64 @ w13q[inter:].T
    h = a * _sig(a) * v
    return _fp8_act(h) @ w2q.T
