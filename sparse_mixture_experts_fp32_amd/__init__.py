"""MI355X (gfx950) mixture-of-experts feed-forward layer: HIP kernels behind a C ABI
(include/moe.h, libmoe.so) and a thin ctypes binding with the same function names."""
from .moe import (  # noqa: F401
    LIB_PATH, MOE_BF16, MOE_ERR_ARG, MOE_ERR_HIP, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
    MOE_F32, MOE_OK, MOE_ROUTER_SIGMOID_SHARED, MOE_ROUTER_SOFTMAX_TOPK, MoEError,
    header_functions, load_library, make_config, moe_combine, moe_config_t, moe_forward,
    moe_forward_mxfp4, moe_forward_rmsnorm, moe_forward_static,
    MOE_STATIC_SCRATCH_BYTES, moe_grouped_swiglu, moe_grouped_swiglu_mxfp4,
    moe_mxfp4_pack_scales, moe_mxfp4_scales_bytes, moe_permute, moe_rmsnorm, moe_route,
    moe_workspace_size, status_str,
)
