"""Pins of the oracle's number formats against torch's CPU casts (library
routines) and against the OCP E4M3FN definition's fixed points."""

import numpy as np
import pytest
import torch

from oracle import numerics as nx


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, 4096, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]            # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(nx.bf16_to_f64(bits), ref)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(4096), rng.standard_normal(64) * 1e-30,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)])])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(nx.bf16_round_f64(x.astype(np.float32).astype(np.float64)), ref)


def _torch_e4m3(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_fixed_points():
    vals = np.array([1.0625, 1.1875, 2.0 ** -10, 464.0, 448.0, 1000.0, -1000.0, 2.0 ** -9,
                     1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9, 0.0, -0.0, 240.0, 256.0, 272.0], np.float32)
    codes = nx.e4m3_encode(vals)
    dec = nx.e4m3_decode(codes)
    assert dec.tolist()[:6] == [1.0, 1.25, 0.0, 448.0, 448.0, 448.0]
    assert dec[6] == -448.0
    assert dec[7] == 2.0 ** -9 and dec[8] == 2.0 * 2.0 ** -9 and dec[9] == 2.0 * 2.0 ** -9
    assert codes[10] == 0x00 and codes[11] == 0x80
    assert dec[12] == 240.0 and dec[13] == 256.0 and dec[14] == 256.0   # 272 ties to even (256)
    assert codes[4] == 0x7E                                                # 448 = S.1111.110


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = nx.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000),
        rng.standard_normal(20000) * 2.0 ** -8,          # subnormal range
        # exact midpoints between neighbouring codes (ties)
        (nx.e4m3_decode(np.arange(0, 126, dtype=np.uint8))[:-1] +
         nx.e4m3_decode(np.arange(1, 126, dtype=np.uint8))) / 2,
    ]).astype(np.float32)
    assert np.array_equal(nx.e4m3_encode(x), _torch_e4m3(x))


def test_quant_dequant_error_bound():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((16, 256)) * np.exp(rng.uniform(-3, 3, (16, 1)))).astype(np.float32)
    codes, scale = nx.quant_act_1x128(x)
    y = nx.dequant_act(codes, scale)
    xs = x.astype(np.float64) / np.repeat(scale.astype(np.float64), 128, axis=1)
    normal = np.abs(xs) >= 2.0 ** -6
    rel = np.abs(y - x)[normal] / np.abs(x.astype(np.float64))[normal]
    assert rel.max() <= 2.0 ** -4
    # the largest magnitude of each tile maps to (or next to) 448
    assert np.all(np.abs(nx.e4m3_decode(codes)).reshape(16, 2, 128).max(axis=2) == 448.0)


def test_weight_block_scales():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((256, 384)).astype(np.float32)
    w[3, 200] = 50.0
    codes, scale = nx.quant_w_128x128(w)
    assert scale.shape == (2, 3)
    assert scale[0, 1] == np.float32(np.float32(50.0) / np.float32(448.0))
    y = nx.dequant_w(codes, scale)
    assert np.abs(y - w).max() <= 2.0 ** -4 * np.abs(w).max()


def test_zero_tile_scale_is_one():
    codes, scale = nx.quant_act_1x128(np.zeros((2, 128), np.float32))
    assert scale.tolist() == [[1.0], [1.0]] and not codes.any()
