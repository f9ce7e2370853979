"""MI355X-native quantized MoE layer: a C-ABI HIP library (libqmoe.so, declared
in include/qmoe.h) and its thin ctypes binding."""
from .binding import (  # noqa: F401
    MoeConfig, MoeQExperts, MoeQProj, QmoeError, lib, make_config, qexperts, status_string,
    moe_workspace_size, workspace, moe_route, moe_permute, moe_expert_ffn_q4, moe_combine,
    moe_layer, moe_layer_trace, MoeTrace, MOE_TRACE_MAX, MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL,
    MOE_ERR_HIP, MOE_WFMT_INT4_G32_F16, MOE_WFMT_NVFP4, MOE_OUT_F32, MOE_OUT_BF16,
    MOE_WFMT_INT4_ROW_F32, MOE_WFMT_INT8_ROW_F32, MOE_WFMT_INT2_ROW_F32,
    MOE_MAX_TOKENS, WFMT, moe_layer_flags, MOE_OPT_NO_GRID_WAIT, MOE_OPT_GRID_WAIT_NONE,
    MOE_OPT_INT8_ACTIVATIONS,
    MOE_FLAG_GRID_WAIT_TIMEOUT, moe_layer_noalloc, MOE_NOALLOC_WS_BYTES,
    MoeCacheStats, moe_cache_create, moe_cache_destroy, moe_layer_cached, moe_cache_prefetch,
    moe_cache_pin, moe_cache_unpin_all, moe_cache_get_stats, moe_cache_slot_of,
)
