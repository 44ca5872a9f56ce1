"""Dispatch layout, gated combine and bias update on the GPU against the oracle.

The layout is integer work: offsets, row_token, slot_row and counts must be
bit-exact. The combine is checked against the fp64 output equation.
"""

import numpy as np
import pytest
import torch

import expert_routing_router_amd as M
from oracle import numerics as nx, permute, routing
from tests.gpu_util import dev, host, log, rel_l2

pytestmark = pytest.mark.gpu


def _idx_random(rng, T, N, K, skew=False):
    if skew:   # every token takes the same first experts: one hot segment, many empty ones
        return np.tile(np.arange(K), (T, 1))
    return np.stack([rng.choice(N, K, replace=False) for _ in range(T)]).astype(np.int64)


@pytest.mark.parametrize("T,N,K,skew", [(8192, 256, 8, False), (8192, 256, 8, True), (1, 256, 8, False),
                                        (100, 64, 6, False), (4097, 16, 4, False), (64, 16, 16, False)])
def test_permute_bit_exact(T, N, K, skew):
    rng = np.random.default_rng(T + N + K)
    idx = _idx_random(rng, T, N, K, skew)
    desc = M.make_desc(T=T, d=256, n_routed=N, top_k=K, n_shared=0, inter=128)
    ws = torch.empty(M.moe_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    offsets = torch.empty(N + 1, dtype=torch.int32, device="cuda")
    row_token = torch.empty(T * K, dtype=torch.int32, device="cuda")
    slot_row = torch.empty(T * K, dtype=torch.int32, device="cuda")
    counts = torch.empty(N, dtype=torch.int32, device="cuda")
    u = torch.randn((T, 256), device="cuda").to(torch.bfloat16)
    x_perm = torch.empty((T * K, 256), dtype=torch.bfloat16, device="cuda")
    M.moe_permute(desc, dev(idx, "i32"), offsets, row_token, slot_row, ws, counts=counts, u=u,
                  x_perm=x_perm)
    torch.cuda.synchronize()
    o, rt, sr = permute.layout_fast(idx, N)
    assert np.array_equal(host(offsets), o)
    assert np.array_equal(host(row_token), rt)
    assert np.array_equal(host(slot_row), sr)
    assert np.array_equal(host(counts), np.bincount(idx.reshape(-1), minlength=N))
    assert torch.equal(x_perm, u[row_token.long()])


@pytest.mark.parametrize("io,ydt", [("bf16", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("T,d,K,Ns", [(300, 7168, 8, 1), (17, 256, 4, 2), (64, 2048, 6, 0)])
def test_combine(io, ydt, T, d, K, Ns):
    rng = np.random.default_rng(T * d + K)
    R = T * K
    u = rng.standard_normal((T, d)).astype(np.float32)
    y = rng.standard_normal((R, d)).astype(np.float32)
    ys = rng.standard_normal((max(Ns, 1), T, d)).astype(np.float32)
    slot = rng.permutation(R).astype(np.int32)
    gate = rng.uniform(0, 1, (T, K)).astype(np.float32)
    gate /= gate.sum(axis=1, keepdims=True)
    if io == "bf16":
        u, y, ys = (nx.bf16_round_f64(a).astype(np.float32) for a in (u, y, ys))
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    desc = M.make_desc(T=T, d=d, n_routed=16, top_k=K, n_shared=Ns, inter=128, in_dtype=io,
                       router_dtype=io, expert_dtype=ydt)
    out = torch.empty((T, d), dtype=tdt, device="cuda")
    M.moe_combine(desc, torch.from_numpy(u).to("cuda", tdt), torch.from_numpy(y).to("cuda", tdt),
                  dev(slot, "i32"), dev(gate, "f32"), out,
                  y_shared=torch.from_numpy(ys).to("cuda", tdt) if Ns else None)
    torch.cuda.synchronize()
    ref = u.astype(np.float64) + (ys[:Ns].astype(np.float64).sum(axis=0) if Ns else 0)
    ref = ref + np.einsum("tk,tkd->td", gate.astype(np.float64),
                          y.astype(np.float64)[slot.reshape(T, K)])
    err = rel_l2(host(out), ref)
    log("combine", io, T, d, K, Ns, "rel-L2 %.2e" % err)
    assert err < (3e-3 if io == "bf16" else 1e-6)


def test_bias_update_bit_exact():
    rng = np.random.default_rng(9)
    for T, N, K in [(8192, 256, 8), (4096, 64, 6), (3, 256, 8), (64, 16, 4)]:
        counts = np.bincount(rng.integers(0, N, T * K), minlength=N).astype(np.int32)
        counts[0] = T * K // N if (T * K) % N == 0 else counts[0]   # one expert exactly at the mean
        b = rng.uniform(-0.05, 0.05, N).astype(np.float32)
        desc = M.make_desc(T=T, d=256, n_routed=N, top_k=K, n_shared=0, inter=128)
        bd = dev(b, "f32")
        M.moe_update_bias(desc, dev(counts, "i32"), bd)
        torch.cuda.synchronize()
        want = routing.bias_step(counts, b, T, K, 0.001)
        assert np.array_equal(host(bd).view(np.uint32), want.view(np.uint32))


def test_permute_ignores_expert_ids_out_of_range():
    """Entries of topk_idx outside [0, N) get no row (slot_row -1, not counted, not gathered); the
    layout of the rest is the oracle's layout with those entries moved to an extra last expert."""
    T, N, K = 777, 64, 6
    rng = np.random.default_rng(21)
    idx = _idx_random(rng, T, N, K)
    bad = rng.random((T, K)) < 0.05
    idx[bad] = rng.choice([-1, N, N + 7, -(1 << 30)], int(bad.sum()))
    desc = M.make_desc(T=T, d=256, n_routed=N, top_k=K, n_shared=0, inter=128)
    ws = torch.empty(M.moe_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    offsets = torch.empty(N + 1, dtype=torch.int32, device="cuda")
    row_token = torch.full((T * K,), -5, dtype=torch.int32, device="cuda")
    slot_row = torch.empty(T * K, dtype=torch.int32, device="cuda")
    counts = torch.empty(N, dtype=torch.int32, device="cuda")
    u = torch.randn((T, 256), device="cuda").to(torch.bfloat16)
    x_perm = torch.zeros((T * K, 256), dtype=torch.bfloat16, device="cuda")
    M.moe_permute(desc, dev(idx, "i32"), offsets, row_token, slot_row, ws, counts=counts, u=u, x_perm=x_perm)
    torch.cuda.synchronize()
    moved = np.where(bad, N, idx)
    o, rt, sr = permute.layout_fast(moved, N + 1)
    total = int(o[N])
    log("permute with %d ids out of range: %d rows" % (int(bad.sum()), total))
    assert total == T * K - int(bad.sum())
    assert np.array_equal(host(offsets), o[:N + 1])
    assert np.array_equal(host(row_token)[:total], rt[:total])
    assert np.array_equal(host(slot_row), np.where(bad.reshape(-1), -1, sr))
    assert np.array_equal(host(counts), np.bincount(idx[~bad], minlength=N))
    assert torch.equal(x_perm[:total], u[row_token[:total].long()])
    assert not x_perm[total:].float().abs().sum().item()


def test_combine_skips_rows_out_of_range():
    """slot_row entries of -1 (a dropped selection) or outside [0, T*K) add nothing."""
    T, d, K, Ns = 129, 512, 4, 1
    rng = np.random.default_rng(22)
    R = T * K
    u = nx.bf16_round_f64(rng.standard_normal((T, d))).astype(np.float32)
    y = nx.bf16_round_f64(rng.standard_normal((R, d))).astype(np.float32)
    ys = nx.bf16_round_f64(rng.standard_normal((Ns, T, d))).astype(np.float32)
    slot = rng.permutation(R).astype(np.int32)
    bad = rng.random(R) < 0.1
    slot[bad] = rng.choice([-1, R, R + 100, -(1 << 30)], int(bad.sum()))
    gate = rng.uniform(0, 1, (T, K)).astype(np.float32)
    desc = M.make_desc(T=T, d=d, n_routed=16, top_k=K, n_shared=Ns, inter=128)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    M.moe_combine(desc, torch.from_numpy(u).to("cuda", torch.bfloat16), torch.from_numpy(y).to("cuda", torch.bfloat16),
                  dev(slot, "i32"), dev(gate, "f32"), out, y_shared=torch.from_numpy(ys).to("cuda", torch.bfloat16))
    torch.cuda.synchronize()
    g = np.where(bad.reshape(T, K), 0.0, gate.astype(np.float64))
    ref = u.astype(np.float64) + ys[0].astype(np.float64)
    ref = ref + np.einsum("tk,tkd->td", g, y.astype(np.float64)[np.where(bad, 0, slot).reshape(T, K)])
    err = rel_l2(host(out), ref)
    log("combine with %d slots out of range: rel-L2 %.2e" % (int(bad.sum()), err))
    assert err < 3e-3
