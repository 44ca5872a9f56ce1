"""Sequence-wise balance loss (moe_seq_balance_loss) on the GPU against oracle.balance.

f is a count divided once, so it is bit-exact; P and the loss are fp64 sums in
another order than the oracle's, rounded to fp32: they must agree to 2 ulp of fp32.
Inputs: affinities and selections from the oracle's router on seeded tokens
(the V3 shape), plus synthetic edge cases (zero rows, one sequence, one token
per sequence, expert counts that are not a multiple of 64).
"""

import functools

import numpy as np
import pytest
import torch

import expert_routing_router_amd as M
from oracle import balance, numerics as nx, routing
from tests.gpu_util import dev, host, log
from workloads import gen, get_config

pytestmark = pytest.mark.gpu


def _gpu(s32, idx, N, K, seq_len, alpha=balance.ALPHA):
    T = s32.shape[0]
    desc = M.make_desc(T=T, d=256, n_routed=N, top_k=K, n_groups=1, topk_groups=1, group_topk=K,
                       n_shared=0, inter=128)
    n_seq = T // seq_len
    f = torch.empty((n_seq, N), dtype=torch.float32, device="cuda")
    P = torch.empty((n_seq, N), dtype=torch.float32, device="cuda")
    loss = torch.empty(n_seq, dtype=torch.float32, device="cuda")
    ws = torch.empty(M.moe_seq_balance_workspace_bytes(desc, seq_len), dtype=torch.uint8, device="cuda")
    M.moe_seq_balance_loss(desc, seq_len, alpha, dev(s32, "f32"), dev(idx.astype(np.int32), "i32"), loss, ws,
                           f=f, P=P)
    torch.cuda.synchronize()
    return host(f), host(P), host(loss)


def _check(s32, idx, N, K, seq_len, tag):
    f, P, L = _gpu(s32, idx, N, K, seq_len)
    fo, Po, Lo = balance.seq_balance(s32, idx, N, K, seq_len, float(np.float32(balance.ALPHA)))
    assert np.array_equal(f, fo.astype(np.float32))
    ulp = np.spacing(np.float32(1.0)) * 2
    assert np.allclose(P, Po, rtol=ulp, atol=1e-30), np.abs(P - Po).max()
    assert np.allclose(L, Lo, rtol=ulp, atol=0), (L, Lo)
    log(tag, "n_seq", len(L), "loss/alpha range %.4e .. %.4e" % (Lo.min() / balance.ALPHA, Lo.max() / balance.ALPHA))


@functools.lru_cache(maxsize=1)
def _v3_routing():
    cfg = get_config("v3")
    u = nx.to_f64(gen.tokens(cfg, 1), cfg.in_dtype)
    E = nx.to_f64(gen.centroids(cfg), cfg.router_dtype)
    r, s64, s32 = routing.route_tokens(u, E, gen.bias_init(cfg), cfg)
    return cfg, s32, r.idx


@pytest.mark.parametrize("seq_len", [4096, 1024, 8192])
def test_v3_router_outputs(seq_len):
    cfg, s32, idx = _v3_routing()
    _check(s32, idx, cfg.n_routed, cfg.top_k, seq_len, "v3 seq_len %d" % seq_len)


def test_skewed_router_outputs():
    cfg = get_config("skew").with_(T=2048)
    u = nx.to_f64(gen.tokens(cfg, 0), cfg.in_dtype)
    E = nx.to_f64(gen.centroids(cfg), cfg.router_dtype)
    r, s64, s32 = routing.route_tokens(u, E, gen.bias_init(cfg), cfg)
    _check(s32, r.idx, cfg.n_routed, cfg.top_k, 512, "skew")


@pytest.mark.parametrize("N,K,T,seq_len", [(96, 6, 300, 100), (16, 4, 64, 1), (256, 8, 32, 32), (200, 3, 50, 25)])
def test_synthetic_edges(N, K, T, seq_len):
    rng = np.random.default_rng(N * 1000 + T)
    s = rng.uniform(0, 1, (T, N)).astype(np.float32)
    s[0] = 0.0                                   # a token whose affinities sum to 0
    s[1, : N // 2] = 0.0
    idx = np.stack([rng.choice(N, K, replace=False) for _ in range(T)]).astype(np.int32)
    _check(s, idx, N, K, seq_len, "N=%d K=%d T=%d seq_len=%d" % (N, K, T, seq_len))


def test_null_f_and_P_and_empty():
    rng = np.random.default_rng(7)
    T, N, K = 128, 64, 4
    s = rng.uniform(0, 1, (T, N)).astype(np.float32)
    idx = np.stack([rng.choice(N, K, replace=False) for _ in range(T)]).astype(np.int32)
    desc = M.make_desc(T=T, d=256, n_routed=N, top_k=K, n_groups=1, topk_groups=1, group_topk=K,
                       n_shared=0, inter=128)
    loss = torch.empty(2, dtype=torch.float32, device="cuda")
    ws = torch.empty(M.moe_seq_balance_workspace_bytes(desc, 64), dtype=torch.uint8, device="cuda")
    M.moe_seq_balance_loss(desc, 64, balance.ALPHA, dev(s, "f32"), dev(idx, "i32"), loss, ws)
    torch.cuda.synchronize()
    _, _, Lo = balance.seq_balance(s, idx, N, K, 64, float(np.float32(balance.ALPHA)))
    assert np.allclose(host(loss), Lo, rtol=2.4e-7)
    d0 = M.make_desc(T=0, d=256, n_routed=N, top_k=K, n_groups=1, topk_groups=1, group_topk=K, n_shared=0,
                     inter=128)
    M.moe_seq_balance_loss(d0, 1, balance.ALPHA, dev(s, "f32"), dev(idx, "i32"), loss, ws)
