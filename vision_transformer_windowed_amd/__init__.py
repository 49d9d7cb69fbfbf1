"""FlashSwin window attention for AMD MI355X (gfx950).

Exact softmax attention inside M x M windows of a token grid, with Swin's
cyclic shift and region mask and window-local 2D RoPE on Q and K, computed by
hand-written HIP kernels behind the C ABI in include/flashswin.h.  The Python
layer only marshals arguments (see _lib.py); torch provides device memory and
streams.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    FSW_BF16,
    FSW_ERR_HIP,
    FSW_ERR_INVALID_ARG,
    FSW_ERR_SCRATCH,
    FSW_ERR_UNSUPPORTED,
    FSW_ERR_WORKSPACE,
    FSW_F32,
    FSW_OK,
    FlashSwinError,
    LIB_PATH,
    MAX_RANK,
    SCRATCH_BYTES,
    WindowAttention,
    WindowAttentionPacked,
    bwd_workspace_bytes,
    flashswin_status_string,
    flashswin_version,
    flashswin_wattn_bwd,
    flashswin_wattn_bwd_workspace_size,
    flashswin_wattn_bwd_lowrank,
    flashswin_wattn_bwd_lowrank_workspace_size,
    flashswin_wattn_bwd_noalloc,
    flashswin_wattn_bwd_packed,
    flashswin_wattn_bwd_packed_stats,
    flashswin_wattn_bwd_stats,
    flashswin_wattn_fwd,
    flashswin_wattn_fwd_lowrank,
    flashswin_wattn_fwd_materialized,
    flashswin_wattn_fwd_materialized_workspace_size,
    flashswin_wattn_fwd_packed,
    flashswin_wattn_fwd_packed_stats,
    flashswin_wattn_fwd_stats,
    flashswin_wattn_stats_bytes,
    load,
    new_stats,
    wattn_bwd,
    wattn_bwd_lowrank,
    wattn_bwd_packed,
    wattn_fwd,
    wattn_fwd_lowrank,
    wattn_fwd_materialized,
    wattn_fwd_packed,
    window_attention,
    window_attention_packed,
)
