"""Grouped SwiGLU experts (moe_expert_ffn) on the GPU against the fp64 oracle.

Segments are ragged on purpose: empty experts, a single row, rows around the
32-row MFMA block and the 256/320-row m-tile edges, and one large segment that
needs several m-tiles; rows are gathered through row_token (random token ids,
with repeats across experts, as after routing).
"""

import numpy as np
import pytest
import torch

import expert_routing_router_amd as M
from oracle import ffn, numerics as nx
from tests.gpu_util import dev, host, log, rel_l2
from workloads import gen

pytestmark = pytest.mark.gpu

COUNTS = [0, 1, 31, 32, 33, 255, 256, 257, 319, 320, 321, 0, 700, 5]


def _weights(rng, n, inter, d, wdtype):
    w13 = (rng.standard_normal((n, 2 * inter, d)) / np.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((n, d, inter)) / np.sqrt(d)).astype(np.float32)
    if wdtype == "bf16":
        return gen.f32_to_bf16_bits(w13), gen.f32_to_bf16_bits(w2)
    return w13, w2


@pytest.mark.parametrize("dtype,d,inter", [("bf16", 256, 128), ("bf16", 1024, 384), ("f32", 256, 96),
                                           ("bf16", 7168, 2048)])
def test_grouped_swiglu(dtype, d, inter):
    rng = np.random.default_rng(d + inter)
    counts = COUNTS if d < 7168 else [0, 250, 262, 1]
    n = len(counts)
    rows = sum(counts)
    T = 600
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_token = rng.integers(0, T, rows).astype(np.int32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    if dtype == "bf16":
        x = gen.f32_to_bf16_bits(x)
    w13, w2 = _weights(rng, n, inter, d, dtype)
    desc = M.make_desc(T=T, d=d, n_routed=16, top_k=2, n_shared=0, inter=inter, in_dtype=dtype,
                       router_dtype=dtype, expert_dtype=dtype)
    ws = torch.empty(M.moe_expert_ffn_workspace_bytes(desc, n, inter, rows), dtype=torch.uint8, device="cuda")
    y = torch.empty((rows, d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    M.moe_expert_ffn(desc, n, inter, rows, dev(x, dtype), dev(offsets, "i32"), dev(w13, dtype),
                     dev(w2, dtype), y, ws, row_token=dev(row_token, "i32"))
    torch.cuda.synchronize()
    got = host(y)
    x64 = nx.to_f64(x, dtype)
    worst = 0.0
    for e in range(n):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        ref = ffn.swiglu(x64[row_token[lo:hi]], nx.to_f64(w13[e], dtype), nx.to_f64(w2[e], dtype))
        err = rel_l2(got[lo:hi], ref)
        worst = max(worst, err)
    log("experts", dtype, d, inter, "worst per-expert rel-L2 %.2e" % worst)
    assert worst < (1e-2 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("d", [512, 384])
def test_grouped_swiglu_direct_rows_and_fp8(d):
    """x read directly (row_token NULL), and the FP8 path against oracle B: d = 512 runs the
    LDS-DMA kernel (256-row tiles), d = 384 (not a multiple of the 256-row weight tile) the
    register-staged 192-row kernel."""
    rng = np.random.default_rng(5)
    inter = 256
    counts = [3, 0, 300, 64, 129]
    n, rows = len(counts), sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = rng.standard_normal((rows, d)).astype(np.float32)
    x[rng.integers(0, rows, 20), rng.integers(0, d, 20)] = 50.0
    w13, w2 = _weights(rng, n, inter, d, "f32")
    desc = M.make_desc(T=rows, d=d, n_routed=16, top_k=1, n_shared=0, inter=inter, in_dtype="bf16",
                       router_dtype="f32", expert_dtype="fp8")
    xb = gen.f32_to_bf16_bits(x)
    xq = torch.empty((rows, d), dtype=torch.uint8, device="cuda")
    xs = torch.empty((rows, d // 128), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(M.MOE_QUANT_ACT_1x128, dev(xb, "bf16"), rows, d, xq, xs)
    q13 = torch.empty((n, 2 * inter, d), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((n, 2 * inter // 128, d // 128), dtype=torch.float32, device="cuda")
    q2 = torch.empty((n, d, inter), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((n, d // 128, inter // 128), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(M.MOE_QUANT_W_128x128, dev(w13.reshape(-1, d), "f32"), n * 2 * inter, d, q13, s13)
    M.moe_quantize_fp8(M.MOE_QUANT_W_128x128, dev(w2.reshape(-1, inter), "f32"), n * d, inter, q2, s2)
    ws = torch.empty(M.moe_expert_ffn_workspace_bytes(desc, n, inter, rows), dtype=torch.uint8, device="cuda")
    y = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn(desc, n, inter, rows, xq, dev(offsets, "i32"), q13, q2, y, ws, x_scale=xs,
                     w13_scale=s13, w2_scale=s2)
    torch.cuda.synchronize()
    # the quantisers are bit-exact against the oracle's encoder
    cq, cs = nx.quant_act_1x128(nx.bf16_to_f64(xb).astype(np.float32))
    assert np.array_equal(host(xq), cq) and np.array_equal(host(xs), cs)
    cw, sw = nx.quant_w_128x128(w13[2])
    assert np.array_equal(host(q13[2]), cw) and np.array_equal(host(s13[2]), sw)
    got = host(y)
    x64 = nx.bf16_to_f64(xb)
    for e in range(n):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        xq64 = nx.dequant_act(*nx.quant_act_1x128(x64[lo:hi].astype(np.float32)))
        refB = ffn._expert(xq64, *ffn.fp8_weights(w13[e].astype(np.float64), w2[e].astype(np.float64)), True)
        refA = ffn.swiglu(x64[lo:hi], w13[e].astype(np.float64), w2[e].astype(np.float64))
        eB, eA, eAB = rel_l2(got[lo:hi], refB), rel_l2(got[lo:hi], refA), rel_l2(refB, refA)
        log("fp8 expert", e, "vs oracle B %.2e" % eB, "vs A %.2e" % eA, "(B vs A %.2e)" % eAB)
        assert eB < 5e-3
        assert eA < eAB * 1.25 + 5e-3


@pytest.mark.parametrize("src_dtype", ["f32", "bf16"])
def test_quant_act_bit_exact_special_tiles(src_dtype):
    """The 1x128 activation quantiser (fp32 source: the FP8 path's H; bf16: u) against the oracle's
    encoder, bit for bit, on tiles with an all-zero row, values in E4M3's subnormal range, signed
    zeros, exact ties between codes, outliers and ordinary normals; rows of 5 tiles, 67 rows."""
    rng = np.random.default_rng(11)
    rows, cols = 67, 640
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[0] = 0.0
    x[1, :128] = -0.0
    x[2] = rng.standard_normal(cols).astype(np.float32) * 1e-3
    x[3, 5] = 448.0                                        # tile amax 448: scale 1, codes of x exactly
    x[3, 6:128] = np.float32(448.0) * np.float32(1.5) / 16  # a tie halfway between two codes
    x[rng.integers(4, rows, 40), rng.integers(0, cols, 40)] = 50.0
    if src_dtype == "bf16":
        bits = gen.f32_to_bf16_bits(x)
        src = dev(bits, "bf16")
        x32 = nx.bf16_to_f64(bits).astype(np.float32)
    else:
        src = dev(x, "f32")
        x32 = x
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(M.MOE_QUANT_ACT_1x128, src, rows, cols, q, s)
    torch.cuda.synchronize()
    cq, cs = nx.quant_act_1x128(x32)
    assert np.array_equal(host(s), cs)
    assert np.array_equal(host(q), cq)


def test_quant_act_codes_dense_sweep():
    """The activation quantiser's E4M3 codes against the oracle's encoder over a dense sweep of
    fp32 values: every 509th bit pattern from 0 to 448 and every 511th from -0 to -448 (E4M3
    subnormals, fp32 denormals and signed zeros included), plus each pair of neighbouring codes'
    midpoint and the fp32 values just either side of it. Each 128-value tile holds 448 first,
    so its scale is exactly 1 and the codes are those of the values themselves."""
    pos = np.arange(0, 0x43E00001, 509, dtype=np.uint64).astype(np.uint32)
    neg = (np.arange(0, 0x43E00001, 511, dtype=np.uint64) | 0x80000000).astype(np.uint32)
    grid = nx.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))            # every finite non-negative code
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))])
    vals = np.concatenate([pos.view(np.float32), neg.view(np.float32), near, -near])
    rows = -(-vals.size // 127)
    body = np.zeros(rows * 127, dtype=np.float32)
    body[:vals.size] = vals
    x = np.concatenate([np.full((rows, 1), 448.0, dtype=np.float32), body.reshape(rows, 127)], axis=1)
    q = torch.empty((rows, 128), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, 1), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(M.MOE_QUANT_ACT_1x128, dev(x, "f32"), rows, 128, q, s)
    torch.cuda.synchronize()
    assert (host(s) == 1.0).all()
    want = nx.e4m3_encode(x)
    got = host(q)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, "first mismatches: %s" % [(float(x[r, c]), int(got[r, c]), int(want[r, c]))
                                                       for r, c in zip(bad[0][:5], bad[1][:5])]


def test_fp8_wide_scale_range_along_k():
    """The FP8 grouped GEMMs with block scales that jump along K: each row's 128-column
    activation tiles are scaled by 2^-10, 1 and 2^10 in turn (the phase shifting from row to
    row) and the 128x128 weight blocks by 2^-5, 1 and 2^5 in a diagonal pattern, so consecutive
    blocks' scale products differ by up to 2^30. The kernel keeps each accumulator in units of
    the current block's scale and rescales it at every block; against oracle B (the same E4M3
    recipe in fp64) the error must stay at the level of ordinary inputs. 320-row tiles (the
    LDS-DMA kernel at MB = 5), d = 1024 (8 blocks along K for the gate/up GEMM), I = 512
    (4 for the down GEMM)."""
    rng = np.random.default_rng(11)
    d, inter = 1024, 512
    counts = [310, 1, 330, 650]
    n, rows = len(counts), sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    kb = np.arange(d) // 128
    x = rng.standard_normal((rows, d)).astype(np.float32)
    x *= np.exp2(10.0 * (((kb[None, :] + np.arange(rows)[:, None]) % 3) - 1)).astype(np.float32)
    w13, w2 = _weights(rng, n, inter, d, "f32")
    w13 *= np.exp2(5.0 * (((np.arange(2 * inter)[:, None] // 128 + kb[None, :]) % 3) - 1)).astype(np.float32)
    ki = np.arange(inter) // 128
    w2 *= np.exp2(5.0 * (((np.arange(d)[:, None] // 128 + ki[None, :]) % 3) - 1)).astype(np.float32)
    desc = M.make_desc(T=rows, d=d, n_routed=16, top_k=1, n_shared=0, inter=inter, in_dtype="bf16",
                       router_dtype="f32", expert_dtype="fp8")
    xb = gen.f32_to_bf16_bits(x)
    xq = torch.empty((rows, d), dtype=torch.uint8, device="cuda")
    xs = torch.empty((rows, d // 128), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(M.MOE_QUANT_ACT_1x128, dev(xb, "bf16"), rows, d, xq, xs)
    q13 = torch.empty((n, 2 * inter, d), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((n, 2 * inter // 128, d // 128), dtype=torch.float32, device="cuda")
    q2 = torch.empty((n, d, inter), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((n, d // 128, inter // 128), dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(M.MOE_QUANT_W_128x128, dev(w13.reshape(-1, d), "f32"), n * 2 * inter, d, q13, s13)
    M.moe_quantize_fp8(M.MOE_QUANT_W_128x128, dev(w2.reshape(-1, inter), "f32"), n * d, inter, q2, s2)
    ws = torch.empty(M.moe_expert_ffn_workspace_bytes(desc, n, inter, rows), dtype=torch.uint8, device="cuda")
    y = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn(desc, n, inter, rows, xq, dev(offsets, "i32"), q13, q2, y, ws, x_scale=xs,
                     w13_scale=s13, w2_scale=s2)
    torch.cuda.synchronize()
    got = host(y)
    assert np.isfinite(got).all()
    x64 = nx.bf16_to_f64(xb)
    for e in range(n):
        lo, hi = offsets[e], offsets[e + 1]
        xq64 = nx.dequant_act(*nx.quant_act_1x128(x64[lo:hi].astype(np.float32)))
        refB = ffn._expert(xq64, *ffn.fp8_weights(w13[e].astype(np.float64), w2[e].astype(np.float64)), True)
        eB = rel_l2(got[lo:hi], refB)
        log("fp8 wide scales, expert", e, "rows", hi - lo, "vs oracle B %.2e" % eB)
        assert eB < 5e-3
