"""MI355X (gfx950) MoE layer with int4/int8 group-quantized experts.

Thin Python binding over the C ABI of libmoe_layer.so (include/moe_layer.h).
All compute runs in the library's HIP kernels; PyTorch only provides device
memory and streams.  Importing this package never falls back to anything else:
if the library is missing, every call raises.
"""

from ._lib import (  # noqa: F401
    MOE_BF16,
    MOE_F32,
    STORE_DIRECT,
    ExpertCache,
    ExpertStore,
    GdnDesc,
    LaunchTimer,
    MoeDesc,
    MoeError,
    blob_bytes,
    clear_launch_events,
    desc_for,
    experts_forward,
    gdn_desc,
    gdn_forward,
    layer_forward,
    layer_forward_chain,
    layer_forward_noalloc,
    layer_forward_scalar,
    layer_forward_staged,
    last_error,
    lib,
    residual_add,
    router_topk,
    stack_forward,
    status_check,
    workspace_bytes,
    workspace_init,
)
