"""MI355X-native AWQ activation-aware scale search and 4-bit packing.

The work runs in libawq_act.so (hand-written HIP for gfx950, C ABI in include/awq_act.h);
this package is a thin ctypes binding with the same entry-point names.
"""
from ._lib import (  # noqa: F401
    AWQ_MAX_ALPHA,
    AWQ_OK,
    AWQ_STAT_EMA_MEAN,
    AWQ_STAT_MAX_ABS,
    AWQ_STAT_MEAN_ABS,
    AWQ_STAT_RMS_RATIO,
    AWQ_W_NONFINITE,
    AwqError,
    LIB_PATH,
    awq_act_stats,
    awq_act_stats_ex,
    awq_act_stats_ex_workspace_bytes,
    awq_act_stats_workspace_bytes,
    awq_clip_search,
    awq_clip_workspace_bytes,
    awq_quantize_pack_clipped,
    awq_hadamard_rotate,
    awq_search_scale_table,
    awq_threshold_scales,
    awq_w4a16_matmul,
    awq_w4a16_workspace_bytes,
    awq_fake_quant_delta,
    awq_quantize_pack,
    awq_search_scales,
    awq_set_profile_events,
    awq_workspace_bytes,
    lib,
    qconfig,
    quantize_layer,
    status_str,
)
