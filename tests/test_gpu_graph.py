"""moe_forward recorded into a HIP graph and replayed.

The forward enqueues only kernels on the caller's stream (no allocation, no
memset, no copy, no synchronisation), so a caller can capture a whole step,
routing, dispatch, both grouped GEMMs, the combine and the bias update, and
replay it on new batches. Each replay is checked bit for bit against the same
step run eagerly, with eager work and host synchronisations between the
replays; the bias update inside the graph advances b exactly as the eager steps
do.
"""

import pytest
import torch

from expert_routing_router_amd.layer import MoELayer
from tests.gpu_util import dev, log
from tests.host_weights import CachedGen
from workloads import gen, get_config

pytestmark = pytest.mark.gpu

NAMES = ("out", "topk_idx", "topk_gate", "counts", "b")


@pytest.mark.parametrize("name,kw", [("mid", dict(T=1024)), ("fp8", dict(T=1024))])
def test_forward_graph_replays_match_eager(name, kw):
    cfg = get_config(name, **kw)
    layer = MoELayer(cfg, CachedGen)
    b0 = gen.bias_init(cfg)
    steps = 4
    us = [dev(gen.tokens(cfg, s), cfg.in_dtype) for s in range(steps)]

    # the eager steps from the initial bias
    b = dev(b0, "f32")
    ref = []
    for s in range(steps):
        layer.forward(us[s], b, update_bias=True)
        torch.cuda.synchronize()
        ref.append([x.clone() for x in (layer.out, layer.idx, layer.gate, layer.counts, b)])

    # one step on static buffers, captured once (capture records, it does not run)
    u_static = us[0].clone()
    b_static = dev(b0, "f32")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        layer.forward(u_static, b_static, update_bias=True)
    torch.cuda.synchronize()
    assert torch.equal(b_static, dev(b0, "f32")), "capture must not execute the step"

    for s in range(steps):
        u_static.copy_(us[s])
        g.replay()
        torch.cuda.synchronize()
        got = (layer.out, layer.idx, layer.gate, layer.counts, b_static)
        for a, e, n in zip(got, ref[s], NAMES):
            assert torch.equal(a, e), "%s step %d: graph replay differs from the eager step in %s" % (name, s, n)
        # eager work between replays: a reduction on the output and a host round trip
        total = float(layer.out.float().abs().sum().item())
        assert total == total
    log(name, kw, "%d graph replays bit-identical to the eager steps" % steps)
