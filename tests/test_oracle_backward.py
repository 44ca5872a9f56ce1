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
