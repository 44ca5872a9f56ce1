"""Host copies of the seeded expert weights for the GPU tests, drawn once per
process and shared by the device layers and the oracle, plus the oracle's
per-expert fp64 weights prepared ahead on a thread pool.

No arithmetic of the layer lives here: weights come from `workloads.gen`
(seeded draws), their fp64 forms from the oracle's own `numerics.to_f64` and
`ffn.fp8_weights`. The thread pool only changes when an expert's weights are
ready, not what the oracle computes with them.
"""

from collections import OrderedDict
from concurrent.futures import ThreadPoolExecutor
import os
import threading

import numpy as np

from oracle import ffn, numerics as nx
from workloads import gen

THREADS = min(16, os.cpu_count() or 1)
_lock = threading.Lock()
_cache = OrderedDict()        # weight-set key -> {("r"|"s", i): (w13, w2)}
_KEEP = 2                     # weight sets kept (a bf16 V3 set is 22.6 GB of host memory)


def _set_key(cfg):
    return (cfg.wid, cfg.d, cfg.inter, cfg.inter_shared, cfg.n_routed, cfg.expert_dtype)


def _cached(cfg):
    """bf16 weight sets are memoised (fp32 masters of FP8 layers are drawn each time)."""
    return cfg.expert_dtype == "bf16"


def _store(cfg):
    key = _set_key(cfg)
    with _lock:
        if key not in _cache:
            while len(_cache) >= _KEEP:
                _cache.popitem(last=False)
            _cache[key] = {}
        _cache.move_to_end(key)
        return _cache[key]


def expert(cfg, kind, i):
    """(w13, w2) canonical arrays of routed expert i (kind "r") or shared expert i ("s")."""
    store = _store(cfg) if _cached(cfg) else None
    k = (kind, i)
    if store is not None:
        with _lock:
            hit = store.get(k)
        if hit is not None:
            return hit
    w = (gen.expert_w13(cfg, i), gen.expert_w2(cfg, i)) if kind == "r" else \
        (gen.shared_w13(cfg, i), gen.shared_w2(cfg, i))
    if store is not None:
        with _lock:
            store[k] = w
    return w


class CachedGen:
    """The `gen` interface MoELayer draws its weights from, backed by the cache."""

    centroids = staticmethod(gen.centroids)

    @staticmethod
    def expert_w13(cfg, e):
        return expert(cfg, "r", e)[0]

    @staticmethod
    def expert_w2(cfg, e):
        return expert(cfg, "r", e)[1]

    @staticmethod
    def shared_w13(cfg, s):
        return expert(cfg, "s", s)[0]

    @staticmethod
    def shared_w2(cfg, s):
        return expert(cfg, "s", s)[1]


def oracle_weights(cfg, experts, fp8=False, ahead=24):
    """A `weights` callable for oracle.ffn.layer: (kind, i) -> fp64 (w13, w2), the
    routed `experts` (ascending, the order the oracle uses them) and the shared
    experts prepared up to `ahead` experts in advance on a thread pool, each
    handed out once."""
    wdt = "bf16" if cfg.expert_dtype == "bf16" else "f32"
    order = [("shared", s) for s in range(cfg.n_shared)] + [("routed", int(e)) for e in sorted(set(experts))]

    def make(job):
        kind, i = job
        a, b = expert(cfg, "s" if kind == "shared" else "r", i)
        a, b = nx.to_f64(a, wdt), nx.to_f64(b, wdt)
        return ffn.fp8_weights(a, b) if fp8 else (a, b)

    pool = ThreadPoolExecutor(THREADS)
    fut = {}
    nxt = [0]

    def fill():
        while nxt[0] < len(order) and len(fut) < ahead:
            job = order[nxt[0]]
            nxt[0] += 1
            fut[job] = pool.submit(make, job)

    fill()

    def get(kind, i):
        job = (kind, int(i))
        if job not in fut:
            raise KeyError("expert %s %d was not announced to oracle_weights" % job)
        w = fut.pop(job).result()
        fill()
        if not fut and nxt[0] >= len(order):
            pool.shutdown(wait=False)
        return w

    return get


def oracle_layer(cfg, u, idx, gate, tokens=None, fp8=False):
    """oracle.ffn.layer over `tokens` (default all) with weights prepared ahead."""
    sel = idx if tokens is None else idx[np.asarray(tokens)]
    w = oracle_weights(cfg, np.unique(sel), fp8=fp8)
    return ffn.layer(cfg, u, idx, gate, None, None, None, None, tokens=tokens, fp8=fp8, weights=w)
