"""Seeded synthetic workloads for the DeepSeekMoE layer.

This package only *draws* inputs: token activations, router centroids, the
initial bias and the expert weights, with the shapes and value distributions of
the layer described in the DeepSeek-V3 Technical Report reading guides
("Método" §2 / "الطريقة" §2 of the xyznot.com pages: 1 shared + 256 routed
experts, 8 active; hidden size 7168 from the zeeklog.com page §3).

It holds none of the layer's arithmetic. It is the one module that both the
HIP path (through the tests and the bench) and the CPU oracle read, so both
sides see bit-identical inputs.
"""

from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    centroids,
    bias_init,
    tokens,
    expert_w13,
    expert_w2,
    shared_w13,
    shared_w2,
    all_weights,
    rng_for,
)
