"""K-blocked expert weights (moe_pack_expert_weights) and the K-blocked H of the
forward. The pack layout is checked against its definition in moe_rocm.h,
written out here with numpy; the forward on blocked copies is checked against
the forward on the row-major weights, which must agree bit for bit (the same
operands reach the same MFMAs in the same order; only where the loads fetch
them from changes). The oracle parity tests of moe_forward run on the blocked
copies too, since MoELayer packs bf16 and FP8 weights by default."""

import numpy as np
import pytest
import torch

import expert_routing_router_amd as M
from expert_routing_router_amd.layer import MoELayer
from tests.gpu_util import dev, log
from tests.host_weights import CachedGen
from tests.test_gpu_forward import layer_for
from workloads import gen, get_config

pytestmark = pytest.mark.gpu


def pack_ref(w, swiglu_i, fp8=False):
    """[n, rows, K] -> [n, tiles, steps, 256, step]: tiles of 256 rows (SwiGLU: gate rows 128t.. then
    up rows swiglu_i + 128t..), steps of 64 bytes (32 bf16 / 64 FP8 elements), row r's 16-byte chunk
    c of 4 at slot c ^ ((r >> 2) & 3)."""
    n, rows, K = w.shape
    step, nch = (64, 4) if fp8 else (32, 4)
    per = 16 // w.dtype.itemsize                                              # elements per chunk
    tiles, steps = rows // 256, K // step
    r = np.arange(256)
    swz = (r >> 2) & 3
    slot_chunk = np.arange(nch)[None, :] ^ swz[:, None]                      # [256, nch]: chunk held by each slot
    out = np.empty((n, tiles, steps, 256, step), w.dtype)
    for t in range(tiles):
        if swiglu_i:
            src = np.concatenate([np.arange(128) + 128 * t, swiglu_i + 128 * t + np.arange(128)])
        else:
            src = 256 * t + np.arange(256)
        tile = w[:, src, :].reshape(n, 256, steps, nch, per)
        g = np.take_along_axis(tile, slot_chunk[None, :, None, :, None], axis=3)
        out[:, t] = g.transpose(0, 2, 1, 3, 4).reshape(n, steps, 256, step)
    return out


@pytest.mark.parametrize("fp8", [False, True])
def test_pack_layout_matches_definition(fp8):
    d, I, Is, N, Ns = 512, 256, 384, 3, 1
    extra = dict(router_dtype="f32", expert_dtype="fp8") if fp8 else {}
    desc = M.make_desc(T=16, d=d, n_routed=N, top_k=2, n_shared=Ns, inter=I, inter_shared=Is, **extra)
    rng = np.random.default_rng(7)
    dt, hi = (np.uint8, 1 << 8) if fp8 else (np.uint16, 1 << 16)
    src = {k: rng.integers(0, hi, size=s, dtype=dt)
           for k, s in (("w13", (N, 2 * I, d)), ("w2", (N, d, I)), ("w13s", (Ns, 2 * Is, d)), ("w2s", (Ns, d, Is)))}
    t = {k: torch.from_numpy(v if fp8 else v.view(np.int16)).cuda() for k, v in src.items()}
    o = {k: torch.empty_like(v) for k, v in t.items()}
    w = M.make_weights(None, t["w13"], t["w2"], t["w13s"], t["w2s"])
    wb = M.make_weights(None, o["w13"], o["w2"], o["w13s"], o["w2s"])
    M.moe_pack_expert_weights(desc, w, wb)
    torch.cuda.synchronize()
    for k, si in (("w13", I), ("w2", 0), ("w13s", Is), ("w2s", 0)):
        got = o[k].cpu().numpy().view(dt).reshape(-1)
        ref = pack_ref(src[k], si, fp8).reshape(-1)
        assert np.array_equal(got, ref), k


def _row_major(weights):
    w = M.MoeWeights.from_buffer_copy(weights)
    w.w13_blk = w.w2_blk = w.w13_shared_blk = w.w2_shared_blk = None
    return w


def _run(layer, weights, u, b, capacity=None):
    out = torch.empty_like(layer.out)
    idx = torch.empty_like(layer.idx)
    gate = torch.empty_like(layer.gate)
    counts = torch.empty_like(layer.counts)
    if capacity is None:
        M.moe_forward(layer.desc, weights, u, b, out, layer.ws, True, idx, gate, counts)
    else:
        ws = torch.empty(M.moe_capacity_workspace_bytes(layer.desc), dtype=torch.uint8, device=u.device)
        keep = torch.empty_like(layer.idx)
        M.moe_forward_capacity(layer.desc, weights, u, b, out, ws, capacity, True, keep, None, idx, gate, counts)
    torch.cuda.synchronize()
    return [x.cpu() for x in (out, idx, gate, counts, b)]


def _same(a, b, tag):
    for name, x, y in zip(("out", "idx", "gate", "counts", "b"), a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), (tag, name)


@pytest.mark.parametrize("name,kw", [("v3", {}), ("mid", {}), ("mid", dict(T=300)), ("fp8", dict(T=2048))])
def test_blocked_forward_bit_identical(name, kw):
    cfg = get_config(name, **kw)
    layer = layer_for(cfg)
    assert layer.blocked, "a bf16 / FP8 layer of this shape keeps K-blocked weights"
    for step in range(2):
        u = dev(gen.tokens(cfg, step), cfg.in_dtype)
        b0 = dev(gen.bias_init(cfg), "f32")
        blk = _run(layer, layer.weights, u, b0.clone())
        row = _run(layer, _row_major(layer.weights), u, b0.clone())
        _same(blk, row, "%s %s step %d" % (name, kw, step))
    log(name, kw, "blocked == row-major")


def test_blocked_capacity_forward_bit_identical():
    """The capped forward runs the shared experts in their own pass (own m-tiles, own blocked H)."""
    cfg = get_config("mid", T=1024, inter_shared=1024)
    layer = MoELayer(cfg, CachedGen)
    assert layer.blocked
    u = dev(gen.tokens(cfg, 0), cfg.in_dtype)
    b0 = dev(gen.bias_init(cfg), "f32")
    cap = (cfg.T * cfg.top_k) // cfg.n_routed
    blk = _run(layer, layer.weights, u, b0.clone(), cap)
    row = _run(layer, _row_major(layer.weights), u, b0.clone(), cap)
    _same(blk, row, "capacity")


def test_unblocked_layer_matches_blocked_layer():
    """A layer built without blocked copies gives the same forward as one with them."""
    cfg = get_config("mid", T=512)
    a = MoELayer(cfg, CachedGen, blocked_weights=False)
    assert not a.blocked
    b = layer_for(cfg)
    assert b.blocked
    u = dev(gen.tokens(cfg, 3), cfg.in_dtype)
    b0 = dev(gen.bias_init(cfg), "f32")
    _same(_run(a, a.weights, u, b0.clone()), _run(b, b.weights, u, b0.clone()), "layers")
