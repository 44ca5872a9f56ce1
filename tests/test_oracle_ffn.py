"""Pins of the oracle's FFN and layer output.

* N_r = 1, K = 1: the layer reduces to u + shared SwiGLU + dense SwiGLU,
  checked against an independently written dense version with torch's CPU
  float64 F.silu (a library routine);
* the literal output equation summed over *all* N_r experts with zero gates
  for the unselected ones equals the oracle's sparse evaluation;
* zero weights give out = u exactly; doubling W2 doubles out - u;
* the order of the K slots does not matter.
"""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import ffn, routing
from workloads import get_config, gen


def _small_cfg(**kw):
    base = dict(T=24, d=64, n_routed=8, top_k=2, n_groups=4, topk_groups=2, group_topk=1,
                n_shared=1, inter=32, inter_shared=48, in_dtype="f32", router_dtype="f32",
                expert_dtype="f32")
    base.update(kw)
    return get_config("tiny", **base)


def _inputs(cfg):
    u = gen.tokens(cfg, 0)
    E = gen.centroids(cfg)
    w13, w2, w13s, w2s = gen.all_weights(cfg, threads=2)
    return u, E, w13, w2, w13s, w2s


def _dense_torch(x, w13, w2):
    x = torch.from_numpy(np.asarray(x, np.float64))
    w13 = torch.from_numpy(np.asarray(w13, np.float64))
    w2 = torch.from_numpy(np.asarray(w2, np.float64))
    inter = w13.shape[0] // 2
    h = F.silu(x @ w13[:inter].T) * (x @ w13[inter:].T)
    return (h @ w2.T).numpy()


def test_single_expert_reduces_to_dense_swiglu():
    cfg = _small_cfg(n_routed=1, top_k=1, n_groups=1, topk_groups=1, group_topk=1)
    u, E, w13, w2, w13s, w2s = _inputs(cfg)
    r, s64, _ = routing.route_tokens(u.astype(np.float64), E.astype(np.float64),
                                     np.zeros(1, np.float32), cfg)
    assert (r.idx == 0).all() and (r.gate == 1.0).all()
    out = ffn.layer(cfg, u, r.idx, r.gate, w13, w2, w13s, w2s)
    ref = u.astype(np.float64) + _dense_torch(u, w13s[0], w2s[0]) + _dense_torch(u, w13[0], w2[0])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_sparse_equals_literal_sum_over_all_experts():
    cfg = _small_cfg()
    u, E, w13, w2, w13s, w2s = _inputs(cfg)
    b = np.random.default_rng(0).uniform(-0.02, 0.02, cfg.n_routed).astype(np.float32)
    r, s64, _ = routing.route_tokens(u.astype(np.float64), E.astype(np.float64), b, cfg)
    out = ffn.layer(cfg, u, r.idx, r.gate, w13, w2, w13s, w2s)
    # g_{i,t} over all experts (zero when unselected), then the equation as printed
    g = np.zeros((cfg.T, cfg.n_routed))
    np.put_along_axis(g, r.idx, r.gate, axis=1)
    lit = u.astype(np.float64) + _dense_torch(u, w13s[0], w2s[0])
    for i in range(cfg.n_routed):
        lit += g[:, i:i + 1] * _dense_torch(u, w13[i], w2[i])
    assert np.allclose(out, lit, rtol=1e-12, atol=1e-12)


def test_zero_weights_give_residual():
    cfg = _small_cfg()
    u, E, w13, w2, w13s, w2s = _inputs(cfg)
    r, _, _ = routing.route_tokens(u.astype(np.float64), E.astype(np.float64),
                                   np.zeros(cfg.n_routed, np.float32), cfg)
    z = [np.zeros_like(a) for a in (w13, w2, w13s, w2s)]
    out = ffn.layer(cfg, u, r.idx, r.gate, *z)
    assert np.array_equal(out, u.astype(np.float64))


def test_doubling_w2_doubles_ffn_output():
    cfg = _small_cfg()
    u, E, w13, w2, w13s, w2s = _inputs(cfg)
    r, _, _ = routing.route_tokens(u.astype(np.float64), E.astype(np.float64),
                                   np.zeros(cfg.n_routed, np.float32), cfg)
    out1 = ffn.layer(cfg, u, r.idx, r.gate, w13, w2, w13s, w2s) - u
    out2 = ffn.layer(cfg, u, r.idx, r.gate, w13, 2 * w2, w13s, 2 * w2s) - u
    # (u + 2y) - u vs 2((u + y) - u): equal up to the rounding of the residual add
    assert np.allclose(out2, 2 * out1, rtol=1e-12, atol=1e-14)


def test_slot_order_invariance():
    cfg = _small_cfg()
    u, E, w13, w2, w13s, w2s = _inputs(cfg)
    r, _, _ = routing.route_tokens(u.astype(np.float64), E.astype(np.float64),
                                   np.zeros(cfg.n_routed, np.float32), cfg)
    out = ffn.layer(cfg, u, r.idx, r.gate, w13, w2, w13s, w2s)
    out_rev = ffn.layer(cfg, u, r.idx[:, ::-1].copy(), r.gate[:, ::-1].copy(), w13, w2, w13s, w2s)
    assert np.allclose(out, out_rev, rtol=1e-13, atol=1e-13)


def test_token_subset_matches_full():
    cfg = _small_cfg()
    u, E, w13, w2, w13s, w2s = _inputs(cfg)
    r, _, _ = routing.route_tokens(u.astype(np.float64), E.astype(np.float64),
                                   np.zeros(cfg.n_routed, np.float32), cfg)
    full = ffn.layer(cfg, u, r.idx, r.gate, w13, w2, w13s, w2s)
    sub = ffn.layer(cfg, u, r.idx, r.gate, w13, w2, w13s, w2s, tokens=[3, 17, 5])
    assert np.allclose(sub, full[[3, 17, 5]], rtol=1e-13, atol=1e-13)


def test_fp8_oracle_b_close_to_a():
    cfg = _small_cfg(d=256, inter=128, inter_shared=128, expert_dtype="fp8", in_dtype="bf16",
                     outlier_frac=0.001)
    u, E, w13, w2, w13s, w2s = _inputs(cfg)
    r, _, _ = routing.route_tokens(ffn.nx.to_f64(u, "bf16"), E.astype(np.float64),
                                   np.zeros(cfg.n_routed, np.float32), cfg)
    a = ffn.layer(cfg, u, r.idx, r.gate, w13, w2, w13s, w2s)
    b = ffn.layer(cfg, u, r.idx, r.gate, w13, w2, w13s, w2s, fp8=True)
    ua = ffn.nx.to_f64(u, "bf16")
    rel = np.linalg.norm(b - a) / np.linalg.norm(a)
    rel_ffn = np.linalg.norm(b - a) / np.linalg.norm(a - ua)
    # E4M3 keeps 3 mantissa bits: per-element rounding of ~2^-4/sqrt(3) RMS on u, W
    # and H gives an FFN-relative error of a few percent, whatever the kernel.
    assert 0.02 < rel_ffn < 0.08 and rel < 0.06
