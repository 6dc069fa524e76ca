"""MI355X-native forward and backward passes of one MoE layer on one GPU's share of experts.

The computation lives in libmoe.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/moe.h).  This package is a thin ctypes binding with the
same names: it turns torch device tensors into pointers and the current torch
stream into a hipStream_t, and nothing else.  There is no fallback: if the
library is not built, every call raises.
"""

from ._lib import (  # noqa: F401
    MOE_BF16,
    MOE_F32,
    MOE_WEIGHTS_OUT_IN,
    MOE_WEIGHTS_IN_OUT,
    MOE_STAGE_COMBINE,
    MOE_STAGE_DISPATCH,
    MOE_STAGE_FFN,
    MOE_STAGE_LAYER,
    MOE_STAGE_ROUTE,
    MOE_STAGE_FFN_BACKWARD,
    MOE_STAGE_ROUTE_BACKWARD,
    MOE_STAGE_LAYER_BACKWARD,
    LayerDesc,
    Saved,
    make_saved,
    RouteOpts,
    MoeError,
    lib,
    lib_path,
    make_desc,
    make_route_opts,
    moe_capacity,
    moe_combine,
    moe_dispatch,
    moe_dispatch_noalloc,
    moe_ep_local_range,
    moe_grouped_ffn,
    moe_last_error,
    moe_layer_forward,
    moe_layer_forward_ex,
    moe_max_pairs,
    moe_profile_events,
    moe_profile_kernel_count,
    moe_profile_kernel_name,
    moe_route,
    moe_route_ex,
    moe_selection_bias_update,
    moe_version,
    moe_grouped_ffn_train,
    moe_layer_forward_train,
    moe_combine_backward,
    moe_grouped_ffn_backward,
    moe_route_backward,
    moe_dispatch_backward,
    moe_layer_backward,
    moe_workspace_size,
)
from .layer import MoELayer  # noqa: F401
