"""MI355X (gfx950) fused-MoE layer: route -> prepare -> align -> experts ->
finalize as hand-written HIP kernels behind the C ABI in include/moe.h.

This package is the thin Python face of libmoe.so (see ``binding``); it
raises ImportError when the library has not been built.
"""

from .binding import (  # noqa: F401
    ForwardGraph,
    MoeError,
    MoeQuantConfig,
    MoeWeights,
    quant_config,
    make_weights,
    moe_align,
    moe_align_capacity,
    moe_experts,
    moe_experts_batched,
    moe_experts_batched_workspace_layout,
    moe_experts_workspace_layout,
    moe_finalize,
    moe_forward,
    moe_forward_monolithic,
    moe_forward_noalloc,
    moe_forward_workspace_bytes,
    moe_pick_block_m,
    moe_prepare,
    moe_route,
    status_str,
    last_error,
    LIB_PATH,
    STAGES,
    NUM_STAGE_EVENTS,
)
