"""MI355X-native DeepSeekMoE layer with auxiliary-loss-free load balancing.

The layer runs in libmoe_rocm.so (hand-written HIP kernels for gfx950) behind
the C ABI declared in include/moe_rocm.h. This package is its Python binding:
`_lib` mirrors the C entry points one to one (same names, marshalling only),
`layer.MoELayer` uploads weights and owns the workspace, `build` compiles the
library in-tree.
"""

from ._lib import (  # noqa: F401
    MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP,
    MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_QUANT_ACT_1x128, MOE_QUANT_W_128x128,
    MoeDesc, MoeError, MoeGrads, MoeRouteOut, MoeWeights,
    lib, header_symbols, make_desc, desc_from_config, make_weights,
    moe_validate, moe_workspace_bytes, moe_expert_ffn_workspace_bytes, moe_route_workspace_bytes,
    moe_route, moe_permute, moe_permute_noalloc, moe_expert_ffn, moe_combine, moe_update_bias, moe_forward,
    moe_quantize_fp8, moe_seq_balance_workspace_bytes, moe_seq_balance_loss,
    moe_transpose_expert_weights, moe_pack_expert_weights, moe_backward_workspace_bytes, moe_backward, make_grads,
    moe_capacity_workspace_bytes, moe_capacity_mask, moe_forward_capacity,
    moe_profile_enable, moe_profile_read, STAGES,
    moe_calibrate_read, moe_calibrate_mfma_bf16, MOE_CAL_MFMA_WAVES,
)
