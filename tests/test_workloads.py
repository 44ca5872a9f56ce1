"""The seeded generators are deterministic, have the stated shapes and
distributions, and their bf16 rounding agrees with torch's cast."""

import numpy as np
import torch

from workloads import gen, get_config


def test_determinism_and_shapes():
    cfg = get_config("tiny")
    assert np.array_equal(gen.tokens(cfg, 0), gen.tokens(cfg, 0))
    assert not np.array_equal(gen.tokens(cfg, 0), gen.tokens(cfg, 1))
    assert gen.tokens(cfg, 0).shape == (64, 256)
    assert gen.centroids(cfg).shape == (16, 256)
    assert gen.expert_w13(cfg, 3).shape == (256, 256)
    assert gen.expert_w2(cfg, 3).shape == (256, 128)
    assert not np.array_equal(gen.expert_w13(cfg, 3), gen.shared_w13(cfg, 0))


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.f32_to_bf16_bits(x), ref)
    assert np.array_equal(gen.bf16_bits_to_f32(ref),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_distributions():
    cfg = get_config("mid", T=512)
    u = gen.bf16_bits_to_f32(gen.tokens(cfg, 0))
    assert abs(u.std() - 1) < 0.02
    w = gen.bf16_bits_to_f32(gen.expert_w13(cfg, 0))
    assert abs(w.std() * np.sqrt(cfg.d) - 1) < 0.02
    b = gen.bias_init(cfg)
    assert b.min() >= -0.01 and b.max() <= 0.01 and b.std() > 0.004


def test_outliers_exact_count():
    cfg = get_config("fp8", T=128, d=1024)
    u = gen.bf16_bits_to_f32(gen.tokens(cfg, 0))
    n = int(round(0.001 * 128 * 1024))
    assert (np.abs(u) == 50).sum() == n
    assert abs((u == 50).sum() - n / 2) < 4 * np.sqrt(n)


def test_skew_centroids_pull_to_first_experts():
    cfg = get_config("skew", T=256, d=512, n_routed=64, n_groups=8)
    E = gen.bf16_bits_to_f32(gen.centroids(cfg))
    n = np.linalg.norm(E, axis=1)
    assert n[0] > 1.5 and n[-1] < 1.2
