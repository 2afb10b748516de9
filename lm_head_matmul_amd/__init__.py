"""FlashSampling for MI355X: fused LM-head matmul + exact Gumbel-max sampling.

The compute lives in libflashsampling.so (hand-written HIP for gfx950, C ABI in
include/flashsampling.h); this package is its Python binding.
"""
from .binding import (  # noqa: F401
    FS_COMBINE_GUMBEL,
    FS_COMBINE_MAX,
    FS_PATH_AUTO,
    FS_PATH_DOT,
    FS_PATH_MFMA,
    FSError,
    LIB_PATH,
    fs_create,
    fs_debug_gumbel_bits,
    fs_debug_gumbel_scan,
    fs_debug_philox,
    fs_destroy,
    fs_fmms_sample,
    fs_fmms_sample_multi,
    fs_fmms_sample_noalloc,
    fs_fmms_sample_top_p,
    fs_fmms_tiling,
    fs_group_combine,
    fs_group_summaries,
    fs_group_summaries_online,
    fs_group_summary,
    fs_last_error,
    fs_profile_next_launch,
    fs_softmax_sample,
    fs_unfused_sample,
    summary_views,
)
