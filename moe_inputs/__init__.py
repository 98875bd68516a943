"""Workload shapes and seeded synthetic inputs for the mixture-of-experts layer.

Shared by the oracle's tests and the GPU path's tests and bench.  Holds no arithmetic of
the layer itself."""
from .configs import CONFIGS, CONFIG_ORDER, EXTRA_ORDER, MoEConfig  # noqa: F401
from .generate import (  # noqa: F401
    EXPERT_TENSORS, MX_BLOCK, f32_to_bf16_bits, fill_expert_mxfp4, fill_expert_tensor,
    make_expert, make_expert_mxfp4, make_inputs, quantize_mxfp4,
    make_logit_offset, make_norm_gain, make_sel_bias, make_w_router, make_x, storage_dtype,
)
