"""Router parity on the GPU against the oracle.

* scores-in mode: with the oracle's fp32 affinities fed in, topk_idx, counts
  and the updated bias are bit-exact, and so are the gates (both sides divide
  the same fp64 sums, the GPU rounds once to fp32);
* end to end (u, E on the GPU): any routing difference is confined to tokens
  whose K-th/(K+1)-th key gap (or M-th/(M+1)-th group-score gap) is below
  1e-6 relative.
"""

import numpy as np
import pytest
import torch

import expert_routing_router_amd as M
from oracle import numerics as nx, routing
from tests.gpu_util import dev, host, log
from workloads import gen, get_config

pytestmark = pytest.mark.gpu


def _desc(T, N, K, G=1, Mg=1, q=None, biased=1, d=256, in_dtype="bf16", router_dtype="bf16"):
    return M.make_desc(T=T, d=d, n_routed=N, top_k=K, n_groups=G, topk_groups=Mg,
                       group_topk=q if q is not None else max(1, K // Mg), n_shared=0, inter=128,
                       in_dtype=in_dtype, router_dtype=router_dtype,
                       expert_dtype="bf16" if in_dtype == "bf16" else "f32",
                       group_score_biased=biased)


def _gpu_route_scores(desc, s32, b32):
    T, N = s32.shape
    K = desc.top_k
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=torch.int32, device="cuda")
    sout = torch.empty((T, N), dtype=torch.float32, device="cuda")
    bd = dev(b32, "f32")
    M.moe_route(desc, bd, idx, gate, counts, scores_in=dev(s32, "f32"), scores_out=sout)
    M.moe_update_bias(desc, counts, bd)
    torch.cuda.synchronize()
    return host(idx), host(gate), host(counts), host(sout), host(bd)


SCORE_CASES = [
    # name, T, N, K, G, M, q, biased, tie_heavy
    ("tiny_shape", 64, 16, 4, 4, 2, 2, 1, False),
    ("mid_shape", 4096, 64, 6, 1, 1, 6, 1, False),
    ("v3_shape", 8192, 256, 8, 8, 4, 2, 1, False),
    ("v3_unbiased_groups", 8192, 256, 8, 8, 4, 2, 0, False),
    ("v3_tie_heavy", 2048, 256, 8, 8, 4, 2, 1, True),
    ("ragged_T", 1000, 64, 6, 4, 2, 3, 1, True),
    ("single_token", 1, 256, 8, 8, 4, 2, 1, False),
    ("k1_g64", 33, 128, 1, 64, 1, 1, 1, True),
    ("q3_groups", 257, 96, 6, 6, 2, 3, 1, False),
    ("all_experts", 50, 16, 16, 1, 1, 16, 1, True),
    # group sizes S = N/G: powers of two up to 64 are scored by segmented cross-lane reductions
    # (S = 64 spans a whole 64-lane slot), other sizes by a lane per group
    ("s64_groups", 777, 256, 8, 4, 2, 4, 1, False),
    ("s64_groups_ties", 300, 256, 8, 4, 2, 4, 1, True),
    ("s8_groups_ties", 500, 64, 6, 8, 3, 2, 1, True),
    ("s1_groups", 40, 16, 4, 16, 4, 1, 1, True),
    ("s32_partial_slot", 400, 96, 4, 3, 2, 2, 1, True),
    ("s24_lane_per_group", 300, 96, 6, 4, 2, 3, 1, True),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_scores_in_bit_exact(case):
    name, T, N, K, G, Mg, q, biased, ties = case
    rng = np.random.default_rng(abs(hash(name)) % 2 ** 32)
    if ties:
        s = rng.choice(np.array([0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 1.0, 0.0], np.float32), (T, N))
        b = rng.choice(np.array([0, 0.125, -0.125, 0.25, -0.0], np.float32), N)
    else:
        s = rng.uniform(0, 1, (T, N)).astype(np.float32)
        b = rng.uniform(-0.01, 0.01, N).astype(np.float32)
    desc = _desc(T, N, K, G, Mg, q, biased)
    r = routing.select(s, b, K, G, Mg, q, biased)
    idx, gate, counts, sout, b1 = _gpu_route_scores(desc, s, b)
    assert np.array_equal(sout, s)
    assert np.array_equal(idx, r.idx), np.nonzero((idx != r.idx).any(axis=1))[0][:10]
    assert np.array_equal(counts, r.counts)
    assert np.array_equal(gate, r.gate.astype(np.float32))
    want_b = routing.bias_step(r.counts, b, T, K, 0.001)
    assert np.array_equal(b1.view(np.uint32), want_b.view(np.uint32))


def test_scores_in_nan_and_zero_sum_gates():
    """Scores-in at the V3 routing shape with degenerate affinities: a NaN
    affinity ranks after every number (it is never chosen while enough numbers
    remain), and a token whose selected affinities are all zero gets gates 1/K
    (the zero-sum reading). Bit-exact against the oracle, as the other cases."""
    T, N, K, G, Mg, q = 512, 256, 8, 8, 4, 2
    rng = np.random.default_rng(77)
    s = rng.uniform(0, 1, (T, N)).astype(np.float32)
    b = rng.uniform(-0.01, 0.01, N).astype(np.float32)
    b[:K] = np.float32(0.5)                           # experts 0..K-1 lead on the biased key
    for t in range(50):                               # 1..3 NaNs, one at the row's best expert
        cols = rng.choice(N, rng.integers(1, 4), replace=False)
        s[t, cols] = np.nan
        s[t, np.nanargmax(s[t] + b)] = np.nan
    s[50:60] = 0.0                                    # all zero: the bias alone routes
    s[60:70] = rng.uniform(0, 0.4, (10, N)).astype(np.float32)
    s[60:70, :K] = 0.0                                # the K selected have zero affinity
    desc = _desc(T, N, K, G, Mg, q)
    r = routing.select(s, b, K, G, Mg, q, 1)
    assert (r.gate[50:70] == 1.0 / K).all() and not np.isnan(r.gate).any()
    idx, gate, counts, sout, b1 = _gpu_route_scores(desc, s, b)
    assert np.array_equal(idx, r.idx), np.nonzero((idx != r.idx).any(axis=1))[0][:10]
    assert np.array_equal(counts, r.counts)
    assert np.array_equal(gate, r.gate.astype(np.float32))
    assert np.array_equal(b1.view(np.uint32), routing.bias_step(r.counts, b, T, K, 0.001).view(np.uint32))


def test_scores_from_oracle_logits_tiny_and_mid():
    for name in ("tiny", "mid"):
        cfg = get_config(name)
        u = nx.to_f64(gen.tokens(cfg, 0), cfg.in_dtype)
        E = nx.to_f64(gen.centroids(cfg), cfg.router_dtype)
        b = gen.bias_init(cfg)
        s32 = routing.sigmoid(routing.logits(u, E)).astype(np.float32)
        desc = M.desc_from_config(cfg)
        r = routing.select(s32, b, cfg.top_k, cfg.n_groups, cfg.topk_groups, cfg.group_topk)
        idx, gate, counts, _, b1 = _gpu_route_scores(desc, s32, b)
        assert np.array_equal(idx, r.idx) and np.array_equal(counts, r.counts)
        assert np.array_equal(b1, routing.bias_step(r.counts, b, cfg.T, cfg.top_k))
        log(name, "scores-in routing bit-exact")


def _e2e(cfg, step=0, b=None, T=None):
    if T is not None:
        cfg = cfg.with_(T=T)
    u = gen.tokens(cfg, step)
    E = gen.centroids(cfg)
    b = gen.bias_init(cfg) if b is None else b
    desc = M.desc_from_config(cfg)
    T, N, K = cfg.T, cfg.n_routed, cfg.top_k
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=torch.int32, device="cuda")
    sout = torch.empty((T, N), dtype=torch.float32, device="cuda")
    M.moe_route(desc, dev(b, "f32"), idx, gate, counts, u=dev(u, cfg.in_dtype),
                E=dev(E, cfg.router_dtype), scores_out=sout)
    torch.cuda.synchronize()
    r, s64, s32 = routing.route_tokens(nx.to_f64(u, cfg.in_dtype), nx.to_f64(E, cfg.router_dtype), b, cfg)
    kgap, ggap = routing.near_tie_gaps(r, K, cfg.topk_groups)
    return r, s64, s32, kgap, ggap, host(idx), host(gate), host(counts), host(sout)


# V3-shaped routers outside the lane-major selection's fast cases: 4 groups of 64 with the
# top-3 group score (the split-K logits, then the one-expert-per-lane selection on the slice
# partials), and no group limit (the lane-major selection with G = 1). Two other widths take
# the split-K logits through other slicings of d: 1024 over 8 slices of one 128-element chunk
# (two stages each) for 300 tokens, 384 over 3 slices for 1000 tokens (a ragged token block).
_ROUTER_VARIANTS = {"v3_g4q3": dict(n_groups=4, topk_groups=2, group_topk=3),
                    "v3_g1": dict(n_groups=1, topk_groups=1, group_topk=8),
                    "v3_d1024": dict(d=1024),
                    "v3_d384": dict(d=384)}


@pytest.mark.parametrize("name,T", [("tiny", None), ("mid", None), ("v3", None), ("fp8", 2048),
                                    ("skew", 4096), ("v3", 77), ("v3_g4q3", 2048), ("v3_g1", 1000),
                                    ("v3_d1024", 300), ("v3_d384", 1000)])
def test_end_to_end_routing(name, T):
    cfg = get_config("v3").with_(**_ROUTER_VARIANTS[name]) if name in _ROUTER_VARIANTS else get_config(name)
    r, s64, s32, kgap, ggap, idx, gate, counts, sout = _e2e(cfg, T=T)
    # the GPU's fp32 affinities: logit error ~1e-7 absolute, one rounding of the fp64 sigmoid
    serr = np.abs(sout.astype(np.float64) - s64)
    log(name, "max |s_gpu - s_oracle| %.3e (fp32 ulp at 1: %.1e)" % (serr.max(), 2.0 ** -24))
    assert serr.max() < 2.5e-7
    diff = routing_set_diff(idx, r.idx)
    exempt = (kgap < 1e-6) | (ggap < 1e-6)
    log(name, "T=%d" % r.idx.shape[0], "tokens routed to a different expert set:", len(diff),
        "exempt tokens:", int(exempt.sum()))
    explain(diff, exempt, idx, r, kgap, ggap, sout)
    assert exempt[diff].all()
    ok = np.setdiff1d(np.arange(len(idx)), diff)
    check_order_and_gates(idx[ok], gate[ok], sout[ok], r.idx[ok], r.gate[ok], r.key[ok], cfg, s64[ok])
    if len(diff) == 0:
        assert np.array_equal(counts, r.counts)
    assert counts.sum() == r.idx.size


def routing_set_diff(idx_gpu, idx_ref):
    """Tokens whose *set* of selected experts differs (the rank order of near-equal keys is not unique)."""
    return np.nonzero((np.sort(idx_gpu, axis=1) != np.sort(idx_ref, axis=1)).any(axis=1))[0]


def explain(diff, exempt, idx, r, kgap, ggap, sout):
    for t in diff[~exempt[diff]][:5]:
        log("  token", t, "gpu", idx[t].tolist(), "oracle", r.idx[t].tolist(),
            "kgap %.3e ggap %.3e" % (kgap[t], ggap[t]),
            "oracle keys", r.key[t, r.idx[t]].tolist(), "gpu s", sout[t, idx[t]].tolist())


def check_order_and_gates(idx, gate, s_gpu, idx_ref, gate_ref, key_ref, cfg, s64):
    """Same sets; the GPU's rank order is valid (keys non-increasing under the oracle's keys up to
    1e-6 relative); gates agree per expert."""
    o1, o2 = np.argsort(idx, axis=1), np.argsort(idx_ref, axis=1)
    assert np.array_equal(np.take_along_axis(idx, o1, 1), np.take_along_axis(idx_ref, o2, 1))
    g1, g2 = np.take_along_axis(gate, o1, 1), np.take_along_axis(gate_ref, o2, 1)
    assert np.allclose(g1, g2, rtol=2e-6, atol=0)
    k = np.take_along_axis(key_ref.astype(np.float64), idx, 1)
    assert (k[:, :-1] >= k[:, 1:] - 1e-6 * np.abs(k[:, 1:])).all()


def test_bias_trajectory_200_steps_scores_in():
    """200 forward+update steps of the skewed router (V3 routing shape, 1024 tokens per step):
    with the oracle's fp32 affinities fed in, the GPU's loads and bias equal the oracle's
    at every step, bit for bit, so the whole balancing trajectory is reproduced."""
    cfg = get_config("skew").with_(T=1024)
    T, N, K = cfg.T, cfg.n_routed, cfg.top_k
    E = nx.to_f64(gen.centroids(cfg), cfg.router_dtype)
    desc = M.desc_from_config(cfg)
    b_ref = gen.bias_init(cfg)
    b_dev = dev(b_ref, "f32")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=torch.int32, device="cuda")
    ratio = []
    for step in range(200):
        u = nx.to_f64(gen.tokens(cfg, step), cfg.in_dtype)
        s32 = routing.sigmoid(routing.logits(u, E)).astype(np.float32)
        r = routing.select(s32, b_ref, K, cfg.n_groups, cfg.topk_groups, cfg.group_topk,
                           cfg.group_score_biased)
        M.moe_route(desc, b_dev, idx, gate, counts, scores_in=dev(s32, "f32"))
        M.moe_update_bias(desc, counts, b_dev)
        torch.cuda.synchronize()
        c = host(counts)
        assert np.array_equal(c, r.counts), step
        assert np.array_equal(host(idx), r.idx), step
        b_ref = routing.bias_step(r.counts, b_ref, T, K, cfg.gamma)
        assert np.array_equal(host(b_dev).view(np.uint32), b_ref.view(np.uint32)), step
        ratio.append(c.max() / c.mean())
    log("skew T=1024 max/mean load: step 0 %.2f, 50 %.2f, 100 %.2f, 150 %.2f, 199 %.2f"
        % tuple(ratio[i] for i in (0, 50, 100, 150, 199)))
    # the balancing moves every expert's bias by gamma per step towards the mean load
    assert np.mean(ratio[-20:]) < np.mean(ratio[:20])


def test_skew_200_steps_v3_fresh_batches():
    """The skewed router at the V3 shape (8192 tokens, a fresh seeded batch every step) for 200
    forward+update steps through moe_route's split-K path. At every step the oracle selects from
    the GPU's fp32 affinities: selections, loads and the updated bias equal the oracle's bit for
    bit. At steps 0 and 199 the affinities themselves are compared with the oracle's fp64 ones."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = get_config("skew")
    T, N, K, steps = cfg.T, cfg.n_routed, cfg.top_k, 200
    desc = M.desc_from_config(cfg)
    E_host = gen.centroids(cfg)
    Ed = dev(E_host, cfg.router_dtype)
    b_ref = gen.bias_init(cfg)
    b_dev = dev(b_ref, "f32")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=torch.int32, device="cuda")
    scores = torch.empty((T, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, M.moe_route_workspace_bytes(desc)), dtype=torch.uint8, device="cuda")
    ratio = []
    with ThreadPoolExecutor(8) as ex:                  # batches drawn ahead, 8 in memory at most
        fut = {s: ex.submit(gen.tokens, cfg, s) for s in range(min(8, steps))}
        for step in range(steps):
            u = fut.pop(step).result()
            if step + 8 < steps:
                fut[step + 8] = ex.submit(gen.tokens, cfg, step + 8)
            M.moe_route(desc, b_dev, idx, gate, counts, u=dev(u, cfg.in_dtype), E=Ed, scores_out=scores, ws=ws)
            M.moe_update_bias(desc, counts, b_dev)
            torch.cuda.synchronize()
            s32 = host(scores)
            r = routing.select(s32, b_ref, K, cfg.n_groups, cfg.topk_groups, cfg.group_topk,
                               cfg.group_score_biased)
            c = host(counts)
            assert np.array_equal(host(idx), r.idx), step
            assert np.array_equal(c, r.counts), step
            b_ref = routing.bias_step(r.counts, b_ref, T, K, cfg.gamma)
            assert np.array_equal(host(b_dev).view(np.uint32), b_ref.view(np.uint32)), step
            if step in (0, steps - 1):
                s64 = routing.sigmoid(routing.logits(nx.to_f64(u, cfg.in_dtype), nx.to_f64(E_host, cfg.router_dtype)))
                err = np.abs(s32.astype(np.float64) - s64).max()
                log("skew V3 step %d: max |s_gpu - s_oracle| %.3e" % (step, err))
                assert err < 2.5e-7
            ratio.append(c.max() / c.mean())
    log("skew V3 max/mean load: step 0 %.2f, 50 %.2f, 100 %.2f, 150 %.2f, 199 %.2f"
        % tuple(ratio[i] for i in (0, 50, 100, 150, 199)))
    assert np.mean(ratio[-20:]) < np.mean(ratio[:20])


@pytest.mark.parametrize("name,T", [("v3", None), ("fp8", 1000), ("mid", 4095), ("skew", 2048)])
def test_forward_routing_matches_moe_route(name, T):
    """moe_forward's topk_idx, gates and loads equal moe_route's bit for bit on the same inputs
    (both run the same router: split-K logits at the V3 shape, the tiled two-phase logits for
    fp32 centroids and for 64 experts)."""
    from tests.test_gpu_forward import layer_for
    cfg = get_config(name)
    if T is not None:
        cfg = cfg.with_(T=T)
    layer = layer_for(cfg)
    u = dev(gen.tokens(cfg, 3), cfg.in_dtype)
    b0 = gen.bias_init(cfg) + np.float32(0.004) * (np.arange(cfg.n_routed) % 3 - 1).astype(np.float32)
    b_fwd = dev(b0, "f32")
    layer.forward(u, b_fwd, update_bias=False)
    desc = M.desc_from_config(cfg)
    idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device="cuda")
    gate = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device="cuda")
    counts = torch.empty(cfg.n_routed, dtype=torch.int32, device="cuda")
    M.moe_route(desc, dev(b0, "f32"), idx, gate, counts, u=u, E=layer.E)
    torch.cuda.synchronize()
    assert np.array_equal(host(layer.idx), host(idx))
    assert np.array_equal(host(layer.gate).view(np.uint32), host(gate).view(np.uint32))
    assert np.array_equal(host(layer.counts), host(counts))
    log(name, "T=%d forward routing == moe_route" % cfg.T)
