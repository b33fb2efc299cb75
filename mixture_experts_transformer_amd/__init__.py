"""MI355X-native forward pass of one routed mixture-of-experts layer, and the
backward of its grouped expert matmuls.

The compute lives in libmoe.so (hand-written gfx950 HIP kernels behind the C ABI
of include/moe.h); this package is its thin Python binding.  Importing it fails
loudly if the library has not been built.
"""
from .moe import (  # noqa: F401
    LayerDesc, MoeError, abi_version, layer_desc, moe_combine, moe_grouped_ffn,
    moe_grouped_ffn_bwd, moe_grouped_ffn_bwd_workspace_size, moe_grouped_ffn_workspace_size,
    moe_layer_fwd, moe_layer_workspace_size, moe_permute, moe_permute_e4m3,
    moe_permute_workspace_size,
    moe_dispatch_pack, moe_dispatch_pack_e4m3, moe_dispatch_pack_workspace_size,
    moe_fp8_scale_update,
    moe_grouped_ffn_e4m3, moe_grouped_ffn_e4m3_workspace_size,
    moe_quantize_e4m3,
    moe_ragged_dot, moe_ragged_dot_dlhs, moe_ragged_dot_drhs, moe_ragged_dot_e4m3, moe_route,
    moe_swiglu_quantize_e4m3, status_str, MOE_COMBINE_KEEP_UNROUTED,
    EV_NAMES, MOE_EV_COUNT, moe_layer_workspace_layout, moe_grouped_ffn_hidden_offset,
    moe_permute_noalloc, MOE_PERMUTE_NOALLOC_SCRATCH_BYTES, MOE_OK, MOE_EINVAL, MOE_ESHAPE,
    MOE_EDTYPE, MOE_EALIGN, MOE_EWORKSPACE, MOE_ELAUNCH)
