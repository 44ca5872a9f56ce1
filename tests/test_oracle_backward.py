"""Pins of oracle.backward (autograd gradients of the layer for a fixed routing)
against central finite differences of the forward oracle's own functions
(routing.logits / routing.sigmoid / ffn.swiglu, fp64), and special cases."""

import numpy as np
import pytest

from oracle import backward, ffn, routing


def _problem(seed, T=7, d=8, N=6, K=2, inter=4, n_shared=1):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, d))
    E = rng.standard_normal((N, d)) / np.sqrt(d)
    idx = np.stack([rng.choice(N, K, replace=False) for _ in range(T)])
    w13 = {e: rng.standard_normal((2 * inter, d)) / np.sqrt(d) for e in range(N)}
    w2 = {e: rng.standard_normal((d, inter)) / np.sqrt(inter) for e in range(N)}
    w13s = [rng.standard_normal((2 * inter, d)) / np.sqrt(d) for _ in range(n_shared)]
    w2s = [rng.standard_normal((d, inter)) / np.sqrt(inter) for _ in range(n_shared)]
    dout = rng.standard_normal((T, d))
    return u, E, idx, w13, w2, w13s, w2s, dout


def _objective(u, E, idx, w13, w2, w13s, w2s, dout):
    """sum(out * dout), the layer output built from the forward oracle's functions."""
    s = routing.sigmoid(routing.logits(u, E))
    sel = np.take_along_axis(s, idx, 1)
    g = sel / sel.sum(axis=1, keepdims=True)
    out = u.copy()
    for a, b in zip(w13s, w2s):
        out += ffn.swiglu(u, a, b)
    for t in range(u.shape[0]):
        for k in range(idx.shape[1]):
            e = idx[t, k]
            out[t] += g[t, k] * ffn.swiglu(u[t:t + 1], w13[e], w2[e])[0]
    return float((out * dout).sum())


def _fd(f, x, pos, h=1e-6):
    x0 = x[pos]
    x[pos] = x0 + h
    fp = f()
    x[pos] = x0 - h
    fm = f()
    x[pos] = x0
    return (fp - fm) / (2 * h)


@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_match_finite_differences(seed):
    u, E, idx, w13, w2, w13s, w2s, dout = _problem(seed)
    gr = backward.layer_grads(u, E, idx, dout, w13, w2, w13s, w2s)
    f = lambda: _objective(u, E, idx, w13, w2, w13s, w2s, dout)
    rng = np.random.default_rng(100 + seed)
    e0 = int(idx[0, 0])
    targets = [("du", u, gr["du"]), ("dE", E, gr["dE"]), ("dw13", w13[e0], gr["dw13"][e0]),
               ("dw2", w2[e0], gr["dw2"][e0]), ("dw13s", w13s[0], gr["dw13s"][0]),
               ("dw2s", w2s[0], gr["dw2s"][0])]
    for name, arr, g in targets:
        for _ in range(6):
            pos = tuple(int(rng.integers(0, n)) for n in arr.shape)
            num = _fd(f, arr, pos)
            assert abs(num - g[pos]) <= 1e-6 * max(1.0, abs(num)), (name, pos, num, g[pos])


def test_unused_expert_has_no_gradient_and_single_expert_gate():
    """N_r = K = 1: the gate is 1 whatever s, so E gets no gradient; du is dout plus the
    two SwiGLU branches' input gradients (checked by finite differences)."""
    u, E, idx, w13, w2, w13s, w2s, dout = _problem(3, N=1, K=1)
    gr = backward.layer_grads(u, E, idx, dout, w13, w2, w13s, w2s)
    assert np.abs(gr["dE"]).max() <= 1e-14      # d(s/s)/ds cancels up to rounding
    f = lambda: _objective(u, E, idx, w13, w2, w13s, w2s, dout)
    for pos in [(0, 0), (3, 5), (6, 7)]:
        assert abs(_fd(f, u, pos) - gr["du"][pos]) <= 1e-6


def test_gradient_is_linear_in_dout():
    u, E, idx, w13, w2, w13s, w2s, dout = _problem(4)
    g1 = backward.layer_grads(u, E, idx, dout, w13, w2, w13s, w2s)
    g2 = backward.layer_grads(u, E, idx, -2.5 * dout, w13, w2, w13s, w2s)
    for k in ("du", "dE"):
        assert np.allclose(g2[k], -2.5 * g1[k], rtol=1e-12, atol=1e-14)


def test_expert_weight_grads_match_finite_differences():
    """expert_weight_grads on the rows that chose expert e, with their gates, gives the
    layer's dW13_e, dW2_e: checked against finite differences of the whole layer objective."""
    u, E, idx, w13, w2, w13s, w2s, dout = _problem(5, T=9)
    f = lambda: _objective(u, E, idx, w13, w2, w13s, w2s, dout)
    s = routing.sigmoid(routing.logits(u, E))
    sel = np.take_along_axis(s, idx, 1)
    g = sel / sel.sum(axis=1, keepdims=True)
    rng = np.random.default_rng(7)
    for e in sorted(set(idx.reshape(-1).tolist()))[:3]:
        rows, ks = np.nonzero(idx == e)
        d13, d2 = backward.expert_weight_grads(u[rows], g[rows, ks], dout[rows], w13[e], w2[e])
        for arr, gr in ((w13[e], d13), (w2[e], d2)):
            for _ in range(5):
                pos = tuple(int(rng.integers(0, n)) for n in arr.shape)
                num = _fd(f, arr, pos)
                assert abs(num - gr[pos]) <= 1e-6 * max(1.0, abs(num)), (e, pos, num, gr[pos])


# ----------------------------------------------------------------------------- FP8 backward
# The FP8 layer's backward (oracle.backward.layer_grads_fp8) runs each expert
# GEMM as the pages' three FP8 GEMMs (pwwt.cn note section 3). Pinned two ways:
#  * with every quantiser the identity it is layer_grads (autograd through the
#    plain equations), so the structure of the backward is the exact one;
#  * one expert linear's Fprop/Dgrad/Wgrad equal an independent construction
#    with torch's float8_e4m3fn cast, on inputs where quantising along the wrong
#    axis, leaving the Dgrad input unquantised or aligning the Wgrad tiles
#    anywhere but at the expert's first row would each be caught.

def test_fp8_backward_without_quantisers_is_the_exact_backward():
    u, E, idx, w13, w2, w13s, w2s, dout = _problem(6, T=9, d=256, inter=128)
    a = backward.layer_grads(u, E, idx, dout, w13, w2, w13s, w2s)
    b = backward.layer_grads_fp8(u, E, idx, dout, w13, w2, w13s, w2s, quantise=False)
    for k in ("du", "dE"):
        assert np.allclose(b[k], a[k], rtol=1e-12, atol=1e-12), k
    for k in ("dw13", "dw2"):
        for e in a[k]:
            assert np.allclose(b[k][e], a[k][e], rtol=1e-12, atol=1e-12), (k, e)
    for k in ("dw13s", "dw2s"):
        for x, y in zip(b[k], a[k]):
            assert np.allclose(x, y, rtol=1e-12, atol=1e-12), k


def _q_torch(x, tr, tc):
    """Quantise-dequantise a float64 numpy [R, C] (R % tr == 0, C % tc == 0) in tr x tc tiles
    with torch's float8_e4m3fn: scale = fl32(amax / 448) (1 for an all-zero tile), RNE, +-448."""
    import torch
    t = torch.from_numpy(np.asarray(x, np.float64)).float()
    R, C = t.shape
    v = t.reshape(R // tr, tr, C // tc, tc)
    amax = v.abs().amax(dim=(1, 3), keepdim=True)
    sc = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (v / sc).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return (q.to(torch.float64) * sc.to(torch.float64)).reshape(R, C).numpy()


def _bf16_torch(a):
    import torch
    return torch.from_numpy(np.asarray(a, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def _fp8_linear_ref(x, w, dy, mutation=None, store=False):
    st = _bf16_torch if store else (lambda a: a)
    x, dy = st(x), st(dy)
    n = x.shape[0]
    pad = (-n) % 128
    if mutation == "wgrad_tiles_unaligned":
        pad_front = 64                          # tiles would start 64 rows before the expert
    else:
        pad_front = 0
    padr = lambda a: np.concatenate([np.zeros((pad_front, a.shape[1])), a,
                                     np.zeros(((-(n + pad_front)) % 128, a.shape[1]))], axis=0)
    y = st(_q_torch(x, 1, 128) @ w.T)
    dx = st((dy if mutation == "dgrad_unquantised" else _q_torch(dy, 1, 128)) @ w)
    if mutation == "wgrad_tiles_along_columns":
        dw = _q_torch(dy, 1, 128).T @ _q_torch(x, 1, 128)
    else:
        dw = (_q_torch(padr(dy), 128, 1).T @ _q_torch(padr(x), 128, 1))
    return y, dx, dw


def test_fp8_linear_matches_independent_recipe():
    import torch
    rng = np.random.default_rng(21)
    n, k, m = 200, 256, 256                     # 200 rows: one full and one partial 128-row tile
    x = rng.standard_normal((n, k)) * (2.0 ** (np.arange(n) % 9 - 4))[:, None]
    x[:, :128] *= 8.0
    dy = rng.standard_normal((n, m)) * (2.0 ** ((np.arange(n) // 37) % 5 - 2))[:, None]
    dy[:, 128:] /= 16.0
    w = _q_torch(rng.standard_normal((m, k)) / 16, 128, 128)      # weights on the E4M3 grid
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    y = backward._Fp8Linear.apply(xt, wt, backward.q_rows, backward.q_cols, lambda a: np.asarray(a, np.float64))
    y.backward(torch.from_numpy(dy))
    y_ref, dx_ref, dw_ref = _fp8_linear_ref(x, w, dy)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(y.detach().numpy(), y_ref) < 1e-12
    assert rel(xt.grad.numpy(), dx_ref) < 1e-12
    assert rel(wt.grad.numpy(), dw_ref) < 1e-12
    # the slips this recipe rules out move the gradients far above rounding (measured:
    # 2.6e-2 with the Dgrad input unquantised, 4.7e-2 with Wgrad tiles along the columns,
    # 2.6e-2 with the Wgrad tiles not aligned at the expert's first row; 0.0 when correct)
    for mut, got, idx in (("dgrad_unquantised", xt.grad.numpy(), 1), ("wgrad_tiles_along_columns", wt.grad.numpy(), 2),
                          ("wgrad_tiles_unaligned", wt.grad.numpy(), 2)):
        bad = _fp8_linear_ref(x, w, dy, mutation=mut)[idx]
        assert rel(got, bad) > 1e-3, mut


def test_fp8_expert_weight_grads_match_the_layer():
    """expert_weight_grads_fp8 on one expert's rows (token order) and gates equals that
    expert's gradients from layer_grads_fp8, whose Wgrad tiles start at the same row."""
    u, E, idx, w13, w2, w13s, w2s, dout = _problem(8, T=300, d=256, N=3, K=2, inter=128)   # ~200 rows each
    ref = backward.layer_grads_fp8(u, E, idx, dout, w13, w2, w13s, w2s)
    s = routing.sigmoid(routing.logits(u, E))
    sel = np.take_along_axis(s, idx, 1)
    g = sel / sel.sum(axis=1, keepdims=True)
    for e in range(3):
        rows, ks = np.nonzero(idx == e)
        assert len(rows) > 0
        d13, d2 = backward.expert_weight_grads_fp8(u[rows], g[rows, ks], dout[rows], w13[e], w2[e])
        assert np.allclose(d13, ref["dw13"][e], rtol=1e-10, atol=1e-12), e
        assert np.allclose(d2, ref["dw2"][e], rtol=1e-10, atol=1e-12), e
    # quantise=False is the exact per-expert gradient
    rows, ks = np.nonzero(idx == 0)
    a = backward.expert_weight_grads(u[rows], g[rows, ks], dout[rows], w13[0], w2[0])
    b = backward.expert_weight_grads_fp8(u[rows], g[rows, ks], dout[rows], w13[0], w2[0], quantise=False)
    assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-14) and np.allclose(a[1], b[1], rtol=1e-12, atol=1e-14)


def test_fp8_linear_bf16_storage_matches_independent_recipe():
    """store="bf16": the GEMM inputs are bf16 tensors (rounded before quantising) and the Fprop
    and Dgrad outputs are rounded to bf16; compared with torch's own bf16 cast around the same
    float8 recipe, and far from the fp64-storage gradients on inputs that are not on the bf16 grid."""
    import torch
    rng = np.random.default_rng(22)
    n, k, m = 200, 256, 256
    x = rng.standard_normal((n, k)) * (2.0 ** (np.arange(n) % 9 - 4))[:, None]
    dy = rng.standard_normal((n, m))
    w = _q_torch(rng.standard_normal((m, k)) / 16, 128, 128)
    _, _, st = backward._rules(True, "bf16")
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    y = backward._Fp8Linear.apply(xt, wt, backward.q_rows, backward.q_cols, st)
    y.backward(torch.from_numpy(dy))
    y_ref, dx_ref, dw_ref = _fp8_linear_ref(x, w, dy, store=True)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    # torch casts fp64 to bf16 through fp32; the oracle rounds fp64 to bf16 directly. They
    # differ only where the fp32 value is an exact bf16 tie that the fp64 value was not.
    xb, dyb = _bf16_torch(x), _bf16_torch(dy)
    for got, ref, pre in ((y.detach().numpy(), y_ref, _q_torch(xb, 1, 128) @ w.T),
                          (xt.grad.numpy(), dx_ref, _q_torch(dyb, 1, 128) @ w)):
        diff = got != ref
        f32 = pre[diff].astype(np.float32)
        assert diff.sum() <= 1e-3 * diff.size
        assert ((f32.view(np.uint32) & 0xFFFF) == 0x8000).all() and (f32 != pre[diff]).all()
    assert rel(wt.grad.numpy(), dw_ref) < 1e-12
    _, dx64, dw64 = _fp8_linear_ref(x, w, dy)
    assert rel(xt.grad.numpy(), dx64) > 1e-3 and rel(wt.grad.numpy(), dw64) > 1e-3
    # bf16 values are left as they are
    v = _bf16_torch(rng.standard_normal(1000))
    assert np.array_equal(st(v), v)


def test_fp8_layer_bf16_storage_without_quantisers_is_near_the_exact_backward():
    """With the quantisers off, bf16 storage only adds bf16 rounding: the gradients stay within a
    few bf16 units of layer_grads, and the structure is unchanged."""
    u, E, idx, w13, w2, w13s, w2s, dout = _problem(9, T=9, d=256, inter=128)
    a = backward.layer_grads(u, E, idx, dout, w13, w2, w13s, w2s)
    b = backward.layer_grads_fp8(u, E, idx, dout, w13, w2, w13s, w2s, quantise=False, store="bf16")
    rel = lambda p, q: np.linalg.norm(p - q) / np.linalg.norm(q)
    assert 1e-5 < rel(b["du"], a["du"]) < 1e-2
    for e in a["dw13"]:
        assert rel(b["dw13"][e], a["dw13"][e]) < 1e-2 and rel(b["dw2"][e], a["dw2"][e]) < 1e-2
