"""MI355X (gfx950) hierarchical local attention: window-first permutation,
2D axial RoPE with scaled low-resolution positions, composite-masked
block-sparse attention, inverse permutation.  Python side of the C ABI in
include/ultragen.h; all compute runs in the library's HIP kernels."""
from ._binding import (  # noqa: F401
    DEBUG_EXPORTED, DEBUG_LIB_PATH, EXPORTED, LIB_PATH, UG_BF16, UG_F32, UG_PLAN_HOST_ONLY, UG_PLAN_NO_LR, Layer, Plan, TrainLayer, UgDesc, UgError, UgInfo,
    UgWarmDesc, ug_warm_start,
    bwd_workspace, debug_bounds, desc_of, lib, make_desc, use_library, ug_attn_bwd, ug_attn_bwd_noalloc, ug_attn_fwd, ug_attn_fwd_lse, ug_attn_fwd_raster,
    ug_last_error, ug_permute, ug_permute_rope, ug_plan, ug_plan_export, ug_plan_export_blocks, ug_plan_export_lr,
    ug_plan_export_queues, ug_plan_free,
    ug_plan_info, ug_permute_rope_bwd, ug_rope2d, ug_rope2d_bwd, ug_status_str, ug_unpermute)
