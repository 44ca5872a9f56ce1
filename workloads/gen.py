"""Seeded generators for the layer's inputs.

Every array is drawn from numpy's PCG64 under a SeedSequence of
[cfg_id, stream, ...]; streams: 1 expert weights, 2 centroids (and the skew
direction), 3 tokens, 4 initial bias, 5 outlier positions/signs.

bf16 inputs are drawn in fp32 and rounded to bf16 with round-to-nearest-even
by the bit routine below; the bf16 arrays (as uint16 bit patterns) are the
canonical inputs that both the GPU and the oracle read. fp32 inputs are the
fp32 draws themselves.
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import MoEConfig

STREAM_WEIGHTS, STREAM_CENTROIDS, STREAM_TOKENS, STREAM_BIAS, STREAM_OUTLIERS = 1, 2, 3, 4, 5


def rng_for(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) for w in words])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, std):
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def _weight_dtype(cfg: MoEConfig) -> str:
    # fp8 layers are drawn as fp32 masters; quantisation is part of the method
    return "bf16" if cfg.expert_dtype == "bf16" else "f32"


def tokens(cfg: MoEConfig, step: int = 0) -> np.ndarray:
    """u [T, d]: N(0,1); bf16 bits or fp32. Optional +-outliers at exact count."""
    rng = rng_for(cfg.cfg_id, STREAM_TOKENS, step)
    u = _normal(rng, (cfg.T, cfg.d), 1.0)
    if cfg.outlier_frac > 0:
        n = int(round(cfg.outlier_frac * cfg.T * cfg.d))
        ro = rng_for(cfg.cfg_id, STREAM_OUTLIERS, step)
        pos = ro.choice(cfg.T * cfg.d, size=n, replace=False)
        sign = np.where(ro.integers(0, 2, size=n) == 1, 1.0, -1.0).astype(np.float32)
        u.reshape(-1)[pos] = sign * np.float32(cfg.outlier_value)
    return _as_dtype(u, cfg.in_dtype)


def centroids(cfg: MoEConfig) -> np.ndarray:
    """E [N_r, d]: N(0, 1/d); the skew workload adds a Zipf-ranked shared direction."""
    rng = rng_for(cfg.wid, STREAM_CENTROIDS, 0)
    e = _normal(rng, (cfg.n_routed, cfg.d), 1.0 / np.sqrt(cfg.d))
    if cfg.centroid_kind == "zipf":
        v = rng_for(cfg.wid, STREAM_CENTROIDS, 1).standard_normal(cfg.d)
        v /= np.linalg.norm(v)
        rank = np.arange(1, cfg.n_routed + 1, dtype=np.float64)
        amp = cfg.zipf_alpha * rank ** (-cfg.zipf_exponent)
        e = (e.astype(np.float64) + amp[:, None] * v[None, :]).astype(np.float32)
    return _as_dtype(e, cfg.router_dtype)


def bias_init(cfg: MoEConfig) -> np.ndarray:
    if cfg.bias_kind == "uniform":
        rng = rng_for(cfg.wid, STREAM_BIAS, 0)
        return rng.uniform(-0.01, 0.01, cfg.n_routed).astype(np.float32)
    return np.zeros(cfg.n_routed, dtype=np.float32)


def _w(cfg, e, m, shape, std):
    rng = rng_for(cfg.wid, STREAM_WEIGHTS, e, m)
    return _as_dtype(_normal(rng, shape, std), _weight_dtype(cfg))


def expert_w13(cfg: MoEConfig, e: int) -> np.ndarray:
    """[2I, d]: rows 0..I-1 gate projection W1, rows I..2I-1 up projection W3."""
    return _w(cfg, e, 0, (2 * cfg.inter, cfg.d), 1.0 / np.sqrt(cfg.d))


def expert_w2(cfg: MoEConfig, e: int) -> np.ndarray:
    """[d, I] down projection."""
    return _w(cfg, e, 1, (cfg.d, cfg.inter), 1.0 / np.sqrt(cfg.d))


def shared_w13(cfg: MoEConfig, s: int) -> np.ndarray:
    return _w(cfg, cfg.n_routed + s, 0, (2 * cfg.inter_shared, cfg.d), 1.0 / np.sqrt(cfg.d))


def shared_w2(cfg: MoEConfig, s: int) -> np.ndarray:
    return _w(cfg, cfg.n_routed + s, 1, (cfg.d, cfg.inter_shared), 1.0 / np.sqrt(cfg.d))


def all_weights(cfg: MoEConfig, threads: int = 0, experts=None):
    """Stacked weights: (w13 [N_r,2I,d], w2 [N_r,d,I], w13s [N_s,2Is,d], w2s [N_s,d,Is]).

    Experts are drawn on a thread pool (numpy releases the GIL while drawing).
    `experts` restricts the routed stack to a subset (others left zero) for
    sampled checks.
    """
    threads = threads or min(16, os.cpu_count() or 1)
    wdt = np.uint16 if _weight_dtype(cfg) == "bf16" else np.float32
    w13 = np.zeros((cfg.n_routed, 2 * cfg.inter, cfg.d), dtype=wdt)
    w2 = np.zeros((cfg.n_routed, cfg.d, cfg.inter), dtype=wdt)
    w13s = np.zeros((cfg.n_shared, 2 * cfg.inter_shared, cfg.d), dtype=wdt)
    w2s = np.zeros((cfg.n_shared, cfg.d, cfg.inter_shared), dtype=wdt)
    todo = list(range(cfg.n_routed)) if experts is None else sorted(set(experts))

    def fill_r(e):
        w13[e] = expert_w13(cfg, e)
        w2[e] = expert_w2(cfg, e)

    def fill_s(s):
        w13s[s] = shared_w13(cfg, s)
        w2s[s] = shared_w2(cfg, s)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill_r, todo))
        list(ex.map(fill_s, range(cfg.n_shared)))
    return w13, w2, w13s, w2s
